// KV compression by learned softmax pooling (page 1, "hybrid attention", CSA step 1 and the HCA
// paragraph; page 4 section 3.1: m = 4 for CSA, m' = 128 for HCA) plus the sliding-window fill
// (page 1, "sliding window": the nearest uncompressed tokens, normed and rotated like entries).
//
// One workgroup of 128 threads per (block, sequence).  Each thread owns 4 of the 512 dims, so every
// token row is read as one coalesced 1 KiB transaction; the pooling weights are a softmax over the
// block's per-token logits held in LDS.  The pooled entry is RMSNorm'd, its last 64 dims rotated to
// the block's last token, and stored as bf16.  The optional indexer key (dI <= 128 dims, one
// thread per dim) is pooled with its own logits and stored as bf16 or as E4M3FN codes + scale.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kThreads = 128;
constexpr int kMaxSpan = 1024;

__device__ __forceinline__ float block_reduce_sum(float v, float* red) {
  v = wave_sum(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  return red[0] + red[1];
}
__device__ __forceinline__ float block_reduce_max(float v, float* red) {
  v = wave_max(v);
  const int w = threadIdx.x / kWave;
  __syncthreads();
  if (lane_id() == 0) red[w] = v;
  __syncthreads();
  return fmaxf(red[0], red[1]);
}

// Softmax weights of n logits into wt[0 .. n).  `first` is this thread's logit j = tid (or -inf),
// already loaded; the rest (n > 128) are read here.
__device__ __forceinline__ void pool_weights(const float* __restrict__ srow, int n, float first, float* wt, float* red) {
  float mx = first;
  if (threadIdx.x < n) wt[threadIdx.x] = first;
  for (int j = threadIdx.x + kThreads; j < n; j += kThreads) {
    const float s = srow[j];
    wt[j] = s;
    mx = fmaxf(mx, s);
  }
  mx = block_reduce_max(mx, red);
  float sum = 0.f;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    const float e = __expf(wt[j] - mx);
    wt[j] = e;
    sum += e;
  }
  sum = block_reduce_sum(sum, red);
  const float inv = 1.0f / sum;
  for (int j = threadIdx.x; j < n; j += kThreads) wt[j] *= inv;
  __syncthreads();
}

constexpr int kPre = 8;    // token rows whose loads are issued before the pooling weights exist

__global__ void __launch_bounds__(kThreads)
compress_kernel(const uint16_t* __restrict__ kv_tok, const float* __restrict__ kv_score,
                const uint16_t* __restrict__ ik_tok, const float* __restrict__ ik_score,
                int T, int64_t tok0, int64_t blk_begin, int m, int ov, int dI,
                const uint16_t* __restrict__ gamma, float eps, RopeFreq rf, int64_t rope_offset,
                uint16_t* __restrict__ kv_out, int64_t kv_ld, int64_t ring_cap,
                void* __restrict__ ik_out, float* __restrict__ ik_scale, int64_t ik_ld, int ik_fp8) {
  __shared__ float wt[kMaxSpan];
  __shared__ float red[4];
  const int b = blockIdx.y;
  const int64_t i = blk_begin + blockIdx.x;
  int64_t lo = i * m - ov;
  if (lo < 0) lo = 0;
  const int64_t hi = (i + 1) * m;
  const int n = (int)(hi - lo);
  const int tid = threadIdx.x;
  const bool has_ik = ik_tok != nullptr;

  // ---- every independent load of the first round, issued together ----
  const float* srow = kv_score + (int64_t)b * T + (lo - tok0);
  const uint16_t* xb = kv_tok + ((int64_t)b * T + (lo - tok0)) * kHeadDim + tid * 4;
  const float s0 = srow[tid < n ? tid : n - 1];
  uint2 pre[kPre];
#pragma unroll
  for (int u = 0; u < kPre; ++u) pre[u] = *reinterpret_cast<const uint2*>(xb + (int64_t)(u < n ? u : n - 1) * kHeadDim);
  const uint2 gm = *reinterpret_cast<const uint2*>(gamma + tid * 4);
  const float* isrow = has_ik ? ik_score + (int64_t)b * T + (lo - tok0) : srow;
  const int dim = tid < dI ? tid : 0;
  const uint16_t* kb = has_ik ? ik_tok + ((int64_t)b * T + (lo - tok0)) * dI + dim : nullptr;
  float is0 = 0.f;
  uint32_t ipre[kPre];
  if (has_ik) {
    is0 = isrow[tid < n ? tid : n - 1];
#pragma unroll
    for (int u = 0; u < kPre; ++u) ipre[u] = kb[(int64_t)(u < n ? u : n - 1) * dI];
  }

  // ---- K=V entry: pool, RMSNorm, RoPE at the block's last token ----
  pool_weights(srow, n, tid < n ? s0 : -INFINITY, wt, red);
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
#pragma unroll
  for (int u = 0; u < kPre; ++u) {
    const float w = u < n ? wt[u] : 0.f;
    a0 += w * bf2f_lo(pre[u].x);
    a1 += w * bf2f_hi(pre[u].x);
    a2 += w * bf2f_lo(pre[u].y);
    a3 += w * bf2f_hi(pre[u].y);
  }
  int j = kPre;
  for (; j + 8 <= n; j += 8) {            // 8 independent row loads in flight
    uint2 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = *reinterpret_cast<const uint2*>(xb + (int64_t)(j + u) * kHeadDim);
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float w = wt[j + u];
      a0 += w * bf2f_lo(v[u].x);
      a1 += w * bf2f_hi(v[u].x);
      a2 += w * bf2f_lo(v[u].y);
      a3 += w * bf2f_hi(v[u].y);
    }
  }
  for (; j < n; ++j) {
    const uint2 v = *reinterpret_cast<const uint2*>(xb + (int64_t)j * kHeadDim);
    const float w = wt[j];
    a0 += w * bf2f_lo(v.x);
    a1 += w * bf2f_hi(v.x);
    a2 += w * bf2f_lo(v.y);
    a3 += w * bf2f_hi(v.y);
  }
  const float ss = block_reduce_sum(a0 * a0 + a1 * a1 + a2 * a2 + a3 * a3, red);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
  float y0 = a0 * rstd * bf2f_lo(gm.x), y1 = a1 * rstd * bf2f_hi(gm.x);
  float y2 = a2 * rstd * bf2f_lo(gm.y), y3 = a3 * rstd * bf2f_hi(gm.y);
  const int d0 = tid * 4;
  if (d0 >= kRopeStart) {
    const double pos = (double)((i + 1) * m - 1 + rope_offset);
    float c, s;
    rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2], &c, &s);
    const float r0 = y0 * c - y1 * s, r1 = y0 * s + y1 * c;
    rope_cs(pos, rf.inv[(d0 - kRopeStart) / 2 + 1], &c, &s);
    const float r2 = y2 * c - y3 * s, r3 = y2 * s + y3 * c;
    y0 = r0; y1 = r1; y2 = r2; y3 = r3;
  }
  const int64_t row = ring_cap > 0 ? (i % ring_cap) : i;
  uint2 o;
  o.x = pack_bf2(y0, y1);
  o.y = pack_bf2(y2, y3);
  *reinterpret_cast<uint2*>(kv_out + ((int64_t)b * kv_ld + row) * kHeadDim + d0) = o;

  if (!has_ik) return;
  // ---- indexer key: pooled with its own logits, no norm, no RoPE ----
  pool_weights(isrow, n, tid < n ? is0 : -INFINITY, wt, red);
  float e = 0.f;
#pragma unroll
  for (int u = 0; u < kPre; ++u) e += (u < n ? wt[u] : 0.f) * bf2f(ipre[u]);
  int jj = kPre;
  for (; jj + 8 <= n; jj += 8) {
    uint32_t v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = kb[(int64_t)(jj + u) * dI];
#pragma unroll
    for (int u = 0; u < 8; ++u) e += wt[jj + u] * bf2f(v[u]);
  }
  for (; jj < n; ++jj) e += wt[jj] * bf2f(kb[(int64_t)jj * dI]);
  if (ik_fp8) {
    const float amax = block_reduce_max(tid < dI ? fabsf(e) : 0.f, red);
    const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
    if (tid < dI) {
      uint8_t* dst = reinterpret_cast<uint8_t*>(ik_out) + ((int64_t)b * ik_ld + i) * dI;
      dst[tid] = (uint8_t)f2e4m3(__fdiv_rn(e, s));
    }
    if (tid == 0) ik_scale[(int64_t)b * ik_ld + i] = s;
  } else if (tid < dI) {
    uint16_t* dst = reinterpret_cast<uint16_t*>(ik_out) + ((int64_t)b * ik_ld + i) * dI;
    dst[tid] = (uint16_t)f2bf(e);
  }
}

}  // namespace

int launch_compress(const CompressArgs& a, hipStream_t stream) {
  dim3 grid((unsigned)a.n_blk, (unsigned)a.B);
  LCS_LAUNCH("compress_kernel", compress_kernel, grid, dim3(kThreads), 0, stream,
             a.kv_tok, a.kv_score, a.ik_tok, a.ik_score, a.T, a.tok0, a.blk_begin, a.m, a.ov, a.dI,
             a.gamma, a.eps, rope_freq(a.theta), a.rope_offset, a.kv_out, a.kv_ld, a.ring_cap, a.ik_out,
             a.ik_scale, a.ik_ld, a.ik_fp8);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
