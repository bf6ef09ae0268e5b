// KV compression by learned softmax pooling (page 1, "hybrid attention", CSA step 1 and the HCA
// paragraph; page 4 section 3.1: m = 4 for CSA, m' = 128 for HCA) plus the sliding-window fill
// (page 1, "sliding window": the nearest uncompressed tokens, normed and rotated like entries).
//
// One workgroup of 512 threads per (block, sequence): four groups of 128 threads, each thread owning
// 4 of the 512 dims (every token row is one coalesced 1 KiB read); group q pools rows q, q + 4, ...
// with all of its row loads issued in one round.  The pooling weights are a softmax over the block's
// per-token logits (K=V and indexer computed together).  Group 0 sums the partials, RMSNorms the
// entry, rotates its last 64 dims to the block's last token and stores bf16; group 1 finishes the
// optional indexer key (dI <= 128 dims, one thread per dim), stored as bf16 or E4M3FN codes + scale.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kDimThreads = 128;          // 4 dims each
constexpr int kGroups = 4;                // row groups: group q pools rows q, q + 4, ...
constexpr int kThreads = kDimThreads * kGroups;
constexpr int kMaxSpan = 1024;            // m + overlap

// Block-wide (512 threads) reductions of two values at once; red: 8 float2.
__device__ __forceinline__ float2 block_max2(float a, float b, float2* red) {
  a = wave_max(a);
  b = wave_max(b);
  if (lane_id() == 0) red[threadIdx.x / kWave] = make_float2(a, b);
  __syncthreads();
  float2 r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) { r.x = fmaxf(r.x, red[w].x); r.y = fmaxf(r.y, red[w].y); }
  __syncthreads();
  return r;
}
__device__ __forceinline__ float2 block_sum2(float a, float b, float2* red) {
  a = wave_sum(a);
  b = wave_sum(b);
  if (lane_id() == 0) red[threadIdx.x / kWave] = make_float2(a, b);
  __syncthreads();
  float2 r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) { r.x += red[w].x; r.y += red[w].y; }
  __syncthreads();
  return r;
}
__device__ __forceinline__ float2 block_sum_max(float a, float b, float2* red) {
  a = wave_sum(a);
  b = wave_max(b);
  if (lane_id() == 0) red[threadIdx.x / kWave] = make_float2(a, b);
  __syncthreads();
  float2 r = red[0];
#pragma unroll
  for (int w = 1; w < kThreads / kWave; ++w) { r.x += red[w].x; r.y = fmaxf(r.y, red[w].y); }
  __syncthreads();
  return r;
}

// ROWS: rows per thread whose loads go out in the first round (chosen from the span, so a short
// block issues no duplicate loads); rows beyond 4 * ROWS are read in batches of 8 afterwards.
template <int ROWS>
__global__ void __launch_bounds__(kThreads)
compress_kernel(const uint16_t* __restrict__ kv_tok, const float* __restrict__ kv_score,
                const uint16_t* __restrict__ ik_tok, const float* __restrict__ ik_score,
                int T, int64_t tok0, int64_t blk_begin, int m, int ov, int dI,
                const uint16_t* __restrict__ gamma, float eps, RopeFreq rf, int64_t rope_offset,
                uint16_t* __restrict__ kv_out, int64_t kv_ld, int64_t ring_cap,
                void* __restrict__ ik_out, float* __restrict__ ik_scale, int64_t ik_ld, int ik_fp8) {
  __shared__ float wt[kMaxSpan];          // pooling weights of the K=V rows
  __shared__ float iwt[kMaxSpan];         // and of the indexer rows
  __shared__ float4 part[kGroups][kDimThreads];
  __shared__ float ipart[kGroups][kDimThreads];
  __shared__ float2 red[kThreads / kWave];
  const int b = blockIdx.y;
  const int64_t i = blk_begin + blockIdx.x;
  int64_t lo = i * m - ov;
  if (lo < 0) lo = 0;
  const int64_t hi = (i + 1) * m;
  const int n = (int)(hi - lo);
  const int tid = threadIdx.x;
  const int q = tid / kDimThreads, t = tid % kDimThreads;
  const bool has_ik = ik_tok != nullptr;

  // ---- one round: logits, this thread's rows (j = q + 4u), gamma; clamped, unconditional loads ----
  const float* srow = kv_score + (int64_t)b * T + (lo - tok0);
  const float* isrow = has_ik ? ik_score + (int64_t)b * T + (lo - tok0) : srow;
  const float s_a = srow[min(tid, n - 1)], s_b = srow[min(tid + kThreads, n - 1)];
  const float is_a = isrow[min(tid, n - 1)], is_b = isrow[min(tid + kThreads, n - 1)];
  const uint16_t* xb = kv_tok + ((int64_t)b * T + (lo - tok0)) * kHeadDim + 4 * t;
  uint2 pre[ROWS];
#pragma unroll
  for (int u = 0; u < ROWS; ++u) pre[u] = *reinterpret_cast<const uint2*>(xb + (int64_t)min(q + kGroups * u, n - 1) * kHeadDim);
  const int dim = t < dI ? t : 0;
  const uint16_t* kb = has_ik ? ik_tok + ((int64_t)b * T + (lo - tok0)) * dI + dim : nullptr;
  uint32_t ipre[ROWS];
  if (has_ik) {
#pragma unroll
    for (int u = 0; u < ROWS; ++u) ipre[u] = kb[(int64_t)min(q + kGroups * u, n - 1) * dI];
  }
  const uint2 gm = *reinterpret_cast<const uint2*>(gamma + 4 * t);

  // ---- pooling weights: softmax over the block's n logits, K=V and indexer together ----
  if (n == 1) {
    if (tid == 0) { wt[0] = 1.f; iwt[0] = 1.f; }
  } else {
    const bool va = tid < n, vb = tid + kThreads < n;
    const float2 mx = block_max2(fmaxf(va ? s_a : -INFINITY, vb ? s_b : -INFINITY),
                                 fmaxf(va ? is_a : -INFINITY, vb ? is_b : -INFINITY), red);
    const float ea = va ? __expf(s_a - mx.x) : 0.f, eb = vb ? __expf(s_b - mx.x) : 0.f;
    const float iea = va ? __expf(is_a - mx.y) : 0.f, ieb = vb ? __expf(is_b - mx.y) : 0.f;
    const float2 sum = block_sum2(ea + eb, iea + ieb, red);
    const float inv = 1.0f / sum.x, iinv = 1.0f / sum.y;
    if (va) { wt[tid] = ea * inv; iwt[tid] = iea * iinv; }
    if (vb) { wt[tid + kThreads] = eb * inv; iwt[tid + kThreads] = ieb * iinv; }
  }
  __syncthreads();

  // ---- this group's partial weighted sums ----
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f, e = 0.f;
#pragma unroll
  for (int u = 0; u < ROWS; ++u) {
    const int j = q + kGroups * u;
    const float w = j < n ? wt[j] : 0.f;
    a0 += w * bf2f_lo(pre[u].x);
    a1 += w * bf2f_hi(pre[u].x);
    a2 += w * bf2f_lo(pre[u].y);
    a3 += w * bf2f_hi(pre[u].y);
    if (has_ik) e += (j < n ? iwt[j] : 0.f) * bf2f(ipre[u]);
  }
  for (int j0 = q + kGroups * ROWS; j0 < n; j0 += kGroups * 8) {   // rows beyond the first round
    uint2 v[8];
    uint32_t iv[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = min(j0 + kGroups * u, n - 1);
      v[u] = *reinterpret_cast<const uint2*>(xb + (int64_t)j * kHeadDim);
      iv[u] = has_ik ? kb[(int64_t)j * dI] : 0u;
    }
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const int j = j0 + kGroups * u;
      const float w = j < n ? wt[j] : 0.f;
      a0 += w * bf2f_lo(v[u].x);
      a1 += w * bf2f_hi(v[u].x);
      a2 += w * bf2f_lo(v[u].y);
      a3 += w * bf2f_hi(v[u].y);
      if (has_ik) e += (j < n ? iwt[j] : 0.f) * bf2f(iv[u]);
    }
  }
  part[q][t] = make_float4(a0, a1, a2, a3);
  ipart[q][t] = e;
  __syncthreads();

  // ---- group 0: the K=V entry (RMSNorm, RoPE at the block's last token); group 1: the indexer key ----
  float4 acc = make_float4(0.f, 0.f, 0.f, 0.f);
  float ie = 0.f;
  if (q == 0) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) { const float4 p = part[g][t]; acc.x += p.x; acc.y += p.y; acc.z += p.z; acc.w += p.w; }
  } else if (q == 1 && has_ik && t < dI) {
#pragma unroll
    for (int g = 0; g < kGroups; ++g) ie += ipart[g][t];
  }
  const float2 ssmx = block_sum_max(q == 0 ? acc.x * acc.x + acc.y * acc.y + acc.z * acc.z + acc.w * acc.w : 0.f,
                                    q == 1 && t < dI ? fabsf(ie) : 0.f, red);
  if (q == 0) {
    const float rstd = 1.0f / sqrtf(ssmx.x * (1.0f / kHeadDim) + eps);
    float y0 = acc.x * rstd * bf2f_lo(gm.x), y1 = acc.y * rstd * bf2f_hi(gm.x);
    float y2 = acc.z * rstd * bf2f_lo(gm.y), y3 = acc.w * rstd * bf2f_hi(gm.y);
    const int d0 = t * 4;
    if (d0 >= kRopeStart) {
      const double pos = (double)((i + 1) * m - 1 + rope_offset);
      float c, sn;
      rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2], &c, &sn);
      const float r0 = y0 * c - y1 * sn, r1 = y0 * sn + y1 * c;
      rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2 + 1], &c, &sn);
      const float r2 = y2 * c - y3 * sn, r3 = y2 * sn + y3 * c;
      y0 = r0; y1 = r1; y2 = r2; y3 = r3;
    }
    const int64_t row = ring_cap > 0 ? (i % ring_cap) : i;
    uint2 o;
    o.x = pack_bf2(y0, y1);
    o.y = pack_bf2(y2, y3);
    *reinterpret_cast<uint2*>(kv_out + ((int64_t)b * kv_ld + row) * kHeadDim + d0) = o;
  } else if (q == 1 && has_ik) {
    // indexer key: pooled with its own logits, no norm, no RoPE
    if (ik_fp8) {
      const float amax = ssmx.y;
      const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
      if (t < dI) {
        uint8_t* dst = reinterpret_cast<uint8_t*>(ik_out) + ((int64_t)b * ik_ld + i) * dI;
        dst[t] = (uint8_t)f2e4m3(__fdiv_rn(ie, sc));
      }
      if (t == 0) ik_scale[(int64_t)b * ik_ld + i] = sc;
    } else if (t < dI) {
      uint16_t* dst = reinterpret_cast<uint16_t*>(ik_out) + ((int64_t)b * ik_ld + i) * dI;
      dst[t] = (uint16_t)f2bf(ie);
    }
  }
}

}  // namespace

int launch_compress(const CompressArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.n_blk, (unsigned)a.B);
  const int span = a.m + a.ov;
#define LCS_COMPRESS(R)                                                                                  \
  LCS_LAUNCH("compress_kernel", compress_kernel<R>, grid, dim3(kThreads), 0, stream, a.kv_tok, a.kv_score, \
             a.ik_tok, a.ik_score, a.T, a.tok0, a.blk_begin, a.m, a.ov, a.dI, a.gamma, a.eps,             \
             rope_freq(a.theta), a.rope_offset, a.kv_out, a.kv_ld, a.ring_cap, a.ik_out, a.ik_scale,      \
             a.ik_ld, a.ik_fp8)
  if (span <= kGroups) LCS_COMPRESS(1);
  else if (span <= 2 * kGroups) LCS_COMPRESS(2);
  else if (span <= 8 * kGroups) LCS_COMPRESS(8);
  else LCS_COMPRESS(32);
#undef LCS_COMPRESS
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
