// Device code of the decode-time token append (the operation is described in decode_append.hip):
// one workgroup's work for one sequence, shared by the append kernel and by the kernel that runs the
// append beside the CSA decode selection.  The calling workgroup runs it with exactly its first 128
// threads (the other waves of a larger workgroup must have exited before the call: the barriers
// inside count the waves still running); red is a 2-float LDS scratch.
#pragma once
#include "common.h"
#include "kernels.h"

namespace lcs {
namespace dapp {

constexpr int kThreads = 128;


__device__ __forceinline__ float block_sum(float v, float* red) {
  v = wave_sum(v);
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  const float r = red[0] + red[1];
  __syncthreads();
  return r;
}
__device__ __forceinline__ float block_max(float v, float* red) {
  v = wave_max(v);
  if (lane_id() == 0) red[threadIdx.x / kWave] = v;
  __syncthreads();
  const float r = fmaxf(red[0], red[1]);
  __syncthreads();
  return r;
}

// RoPE on dims d0 .. d0+3 (d0 >= 448) at position pos; y holds the 4 values.
__device__ __forceinline__ void rope4(float (&y)[4], int d0, double pos, const RopeFreq& rf) {
  if (d0 < kRopeStart) return;
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    float c, s;
    rope_cs(pos, rope_inv(rf, (d0 - kRopeStart) / 2 + p), &c, &s);
    const float a0 = y[2 * p], a1 = y[2 * p + 1];
    y[2 * p] = a0 * c - a1 * s;
    y[2 * p + 1] = a0 * s + a1 * c;
  }
}

// The window row of a token, shared by the append (128 threads, thread x: dims 4x .. 4x+3) and by
// ring_row_wave below (one wave doing the work of threads x and x + 64), so both give the same bits.
__device__ __forceinline__ float sq4(const float (&v)[4]) { return v[0] * v[0] + v[1] * v[1] + v[2] * v[2] + v[3] * v[3]; }
__device__ __forceinline__ void norm_rope4(const float (&v)[4], const float (&g4)[4], float ss, float eps, int d0,
                                           double pos, const RopeFreq& rf, float (&y)[4]) {
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
#pragma unroll
  for (int i = 0; i < 4; ++i) y[i] = v[i] * rstd * g4[i];
  rope4(y, d0, pos, rf);
}
__device__ __forceinline__ float absmax4(const float (&y)[4]) {
  return fmaxf(fmaxf(fabsf(y[0]), fabsf(y[1])), fmaxf(fabsf(y[2]), fabsf(y[3])));
}
__device__ __forceinline__ float row_scale(float amax) { return amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f; }
__device__ __forceinline__ uint32_t codes4(const float (&y)[4], float sc) {
  uint32_t c = 0u;
#pragma unroll
  for (int k = 0; k < 4; ++k) c |= f2e4m3(__fdiv_rn(y[k], sc)) << (8 * k);
  return c;
}

// Row (b, row) of a [B, ld, 512] K=V store from this thread's 4 dims: bf16, or (kv8) E4M3FN codes with
// the row's scale absmax / 448 (block-wide max; every thread must call it).  ok = false: not stored.
__device__ __forceinline__ void store_kv_row(const DecodeAppendArgs& a, void* base, float* scale, int64_t b,
                                             int64_t ld, int64_t row, bool ok, const float (&y)[4], float* red) {
  const int x = threadIdx.x;
  const int64_t off = (b * ld + row) * kHeadDim + 4 * x;
  if (a.kv8) {
    const float sc = row_scale(block_max(absmax4(y), red));
    const uint32_t c = codes4(y, sc);
    if (ok) {
      *reinterpret_cast<uint32_t*>(static_cast<uint8_t*>(base) + off) = c;
      if (x == 0) scale[b * ld + row] = sc;
    }
  } else if (ok) {
    *reinterpret_cast<uint2*>(static_cast<uint16_t*>(base) + off) = make_uint2(pack_bf2(y[0], y[1]), pack_bf2(y[2], y[3]));
  }
}

// Token t's window row of sequence b, RoPE_t(RMSNorm(kv_tok[b])), computed by one wave exactly as the
// append computes and stores it (the reduction in the same order: two 64-lane sums added), into LDS:
// 512 bf16 values, or (kv8) 512 E4M3FN codes and the row scale.  The loads (ring_row_load) are apart
// so that a caller can issue them ahead of its other loads.
struct RingRowIn {
  uint2 raw[2], gm[2];
};
__device__ __forceinline__ void ring_row_load(const DecodeAppendArgs& a, int b, RingRowIn& in) {
  const int l = lane_id();
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int x = l + 64 * h;
    in.raw[h] = *reinterpret_cast<const uint2*>(a.kv_tok + (int64_t)b * kHeadDim + 4 * x);
    in.gm[h] = *reinterpret_cast<const uint2*>(a.gamma + 4 * x);
  }
}
__device__ __forceinline__ void ring_row_compute(const DecodeAppendArgs& a, const RopeFreq& rf, int64_t t,
                                                 const RingRowIn& in, void* s_row, float* s_scale) {
  const int l = lane_id();
  float v[2][4], g4[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    v[h][0] = bf2f_lo(in.raw[h].x); v[h][1] = bf2f_hi(in.raw[h].x);
    v[h][2] = bf2f_lo(in.raw[h].y); v[h][3] = bf2f_hi(in.raw[h].y);
    g4[h][0] = bf2f_lo(in.gm[h].x); g4[h][1] = bf2f_hi(in.gm[h].x);
    g4[h][2] = bf2f_lo(in.gm[h].y); g4[h][3] = bf2f_hi(in.gm[h].y);
  }
  const float ss = wave_sum(sq4(v[0])) + wave_sum(sq4(v[1]));
  float y[2][4];
#pragma unroll
  for (int h = 0; h < 2; ++h) norm_rope4(v[h], g4[h], ss, a.eps, 4 * (l + 64 * h), (double)(t + a.rope_offset), rf, y[h]);
  if (a.kv8) {
    const float sc = row_scale(wave_max(fmaxf(absmax4(y[0]), absmax4(y[1]))));
#pragma unroll
    for (int h = 0; h < 2; ++h) static_cast<uint32_t*>(s_row)[l + 64 * h] = codes4(y[h], sc);
    if (l == 0) *s_scale = sc;
  } else {
#pragma unroll
    for (int h = 0; h < 2; ++h)
      static_cast<uint2*>(s_row)[l + 64 * h] = make_uint2(pack_bf2(y[h][0], y[h][1]), pack_bf2(y[h][2], y[h][3]));
  }
}

// The append of sequence b (threads 0 .. 127 of the calling workgroup).
__device__ __forceinline__ void decode_append_seq(const DecodeAppendArgs& a, const RopeFreq& rf, int b, float* red) {
  const int x = threadIdx.x;
  const int64_t t = a.pos[b];
  if (t < 0) return;                                   // inactive slot of the batch (uniform)
  const bool has_ik = a.ik_tok != nullptr;

  // ---- this token ----
  const uint2 raw = *reinterpret_cast<const uint2*>(a.kv_tok + (int64_t)b * kHeadDim + 4 * x);
  const uint2 gm = *reinterpret_cast<const uint2*>(a.gamma + 4 * x);
  const float s = a.kv_score[b];
  const float v[4] = {bf2f_lo(raw.x), bf2f_hi(raw.x), bf2f_lo(raw.y), bf2f_hi(raw.y)};
  const float g4[4] = {bf2f_lo(gm.x), bf2f_hi(gm.x), bf2f_lo(gm.y), bf2f_hi(gm.y)};
  float iv = 0.f, is = 0.f;
  if (has_ik) {
    iv = x < a.dI ? bf2f(a.ik_tok[(int64_t)b * a.dI + x]) : 0.f;
    is = a.ik_score[b];
  }

  // ---- window ring row t % ring_cap: RoPE_t(RMSNorm(x)) ----
  if (a.win != nullptr) {
    const float ss = block_sum(sq4(v), red);
    float y[4];
    norm_rope4(v, g4, ss, a.eps, 4 * x, (double)(t + a.rope_offset), rf, y);
    store_kv_row(a, a.win, a.win_scale, b, a.win_ld, t % a.ring_cap, true, y, red);
  }

  // ---- pooling state of the blocks containing t: i = t / m and, inside the overlap, i + 1 ----
  const int64_t i = t / a.m;
  const bool in_next = a.ov > 0 && t >= (i + 1) * a.m - a.ov;
  float kv_e[4] = {0.f, 0.f, 0.f, 0.f};                // block i's pooled vector when t ends it
  float ik_e = 0.f;
  const bool ends = t == (i + 1) * a.m - 1;
  // read both slots' running values first: (M, l) is shared by all threads and rewritten below
  float4 o[2];
  float2 mlk[2], mli[2];
  float io[2];
  bool init[2], valid[2];
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    const int64_t j = i + q;
    const int64_t first = j * a.m - a.ov > 0 ? j * a.m - a.ov : 0;
    init[q] = t == first;                                        // the block's first token: fresh state
    const float* st = a.state + ((int64_t)b * 2 + (j & 1)) * kStateFloats;
    o[q] = make_float4(0.f, 0.f, 0.f, 0.f);
    mlk[q] = mli[q] = make_float2(0.f, 0.f);
    io[q] = 0.f;
    // same value in every thread: the decisions below are uniform
    valid[q] = init[q] || __float_as_int(st[kHeadDim + kMaxIdxDim + 4]) == (int32_t)(j + 1);
    if ((q == 0 || in_next) && !init[q] && valid[q]) {
      o[q] = reinterpret_cast<const float4*>(st)[x];
      mlk[q] = *reinterpret_cast<const float2*>(st + kHeadDim + kMaxIdxDim);
      if (has_ik) {
        mli[q] = *reinterpret_cast<const float2*>(st + kHeadDim + kMaxIdxDim + 2);
        io[q] = x < a.dI ? st[kHeadDim + x] : 0.f;
      }
    }
  }
  __syncthreads();
  bool finish = false;
#pragma unroll
  for (int q = 0; q < 2; ++q) {
    if (q == 1 && !in_next) break;
    if (!valid[q]) continue;                                     // block opened before this sequence's first append
    const int64_t j = i + q;
    float* st = a.state + ((int64_t)b * 2 + (j & 1)) * kStateFloats;
    float4 A;
    float Mn, ln, IA = 0.f, IMn = 0.f, Iln = 0.f;
    if (init[q]) {
      A = make_float4(v[0], v[1], v[2], v[3]);
      Mn = s;
      ln = 1.f;
      if (has_ik) { IA = iv; IMn = is; Iln = 1.f; }
    } else {
      Mn = fmaxf(mlk[q].x, s);
      const float fo = __expf(mlk[q].x - Mn), fn = __expf(s - Mn);
      A = make_float4(o[q].x * fo + v[0] * fn, o[q].y * fo + v[1] * fn, o[q].z * fo + v[2] * fn,
                      o[q].w * fo + v[3] * fn);
      ln = mlk[q].y * fo + fn;
      if (has_ik) {
        IMn = fmaxf(mli[q].x, is);
        const float gfo = __expf(mli[q].x - IMn), gfn = __expf(is - IMn);
        IA = io[q] * gfo + iv * gfn;
        Iln = mli[q].y * gfo + gfn;
      }
    }
    if (q == 0 && ends) {                                        // block i is complete
      finish = true;
      const float inv = 1.0f / ln;
      kv_e[0] = A.x * inv; kv_e[1] = A.y * inv; kv_e[2] = A.z * inv; kv_e[3] = A.w * inv;
      if (has_ik) ik_e = IA * (1.0f / Iln);
    } else {                                                     // keep the running state
      reinterpret_cast<float4*>(st)[x] = A;
      if (has_ik && x < a.dI) st[kHeadDim + x] = IA;
      if (x == 0) {
        *reinterpret_cast<float2*>(st + kHeadDim + kMaxIdxDim) = make_float2(Mn, ln);
        if (has_ik) *reinterpret_cast<float2*>(st + kHeadDim + kMaxIdxDim + 2) = make_float2(IMn, Iln);
        if (init[q]) st[kHeadDim + kMaxIdxDim + 4] = __int_as_float((int32_t)(j + 1));
      }
    }
  }
  if (!finish) return;                                          // uniform (t and the tag are)

  // ---- block i's entry: RMSNorm, RoPE at its last token t; indexer key ----
  const float ss = block_sum(kv_e[0] * kv_e[0] + kv_e[1] * kv_e[1] + kv_e[2] * kv_e[2] + kv_e[3] * kv_e[3], red);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + a.eps);
  float y[4];
#pragma unroll
  for (int k = 0; k < 4; ++k) y[k] = kv_e[k] * rstd * g4[k];
  rope4(y, 4 * x, (double)(t + a.rope_offset), rf);
  const int64_t row = a.kv_ring > 0 ? i % a.kv_ring : i;
  store_kv_row(a, a.kv_out, a.kv_scale, b, a.kv_ld, row, row < a.kv_ld, y, red);
  if (!has_ik) return;
  const bool ik_row_ok = i < a.ik_ld;
  if (a.ik_fp8) {
    const float amax = block_max(x < a.dI ? fabsf(ik_e) : 0.f, red);
    const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (ik_row_ok && x < a.dI)
      reinterpret_cast<uint8_t*>(a.ik_out)[((int64_t)b * a.ik_ld + i) * a.dI + x] = (uint8_t)f2e4m3(__fdiv_rn(ik_e, sc));
    if (ik_row_ok && x == 0) a.ik_scale[(int64_t)b * a.ik_ld + i] = sc;
  } else if (ik_row_ok && x < a.dI) {
    reinterpret_cast<uint16_t*>(a.ik_out)[((int64_t)b * a.ik_ld + i) * a.dI + x] = (uint16_t)f2bf(ik_e);
  }
}

}  // namespace dapp
}  // namespace lcs
