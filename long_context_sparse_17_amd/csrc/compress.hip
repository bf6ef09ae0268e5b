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

// Softmax weights of the logits of tokens [lo, hi) (columns lo-tok0 ..) into wt[0 .. hi-lo).
__device__ void pool_weights(const float* __restrict__ score_row, int64_t lo, int64_t hi, int64_t tok0,
                             float* wt, float* red) {
  const int n = (int)(hi - lo);
  float mx = -INFINITY;
  for (int j = threadIdx.x; j < n; j += kThreads) {
    const float s = score_row[lo - tok0 + j];
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

__global__ void __launch_bounds__(kThreads)
compress_kernel(const uint16_t* __restrict__ kv_tok, const float* __restrict__ kv_score,
                const uint16_t* __restrict__ ik_tok, const float* __restrict__ ik_score,
                int T, int64_t tok0, int64_t blk_begin, int m, int ov, int dI,
                const uint16_t* __restrict__ gamma, float eps, float theta, int64_t rope_offset,
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

  // ---- K=V entry: pool, RMSNorm, RoPE at the block's last token ----
  pool_weights(kv_score + (int64_t)b * T, lo, hi, tok0, wt, red);
  const uint16_t* xb = kv_tok + ((int64_t)b * T + (lo - tok0)) * kHeadDim + tid * 4;
  float a0 = 0.f, a1 = 0.f, a2 = 0.f, a3 = 0.f;
  for (int j = 0; j < n; ++j) {
    const uint2 v = *reinterpret_cast<const uint2*>(xb + (int64_t)j * kHeadDim);
    const float w = wt[j];
    a0 += w * bf2f_lo(v.x);
    a1 += w * bf2f_hi(v.x);
    a2 += w * bf2f_lo(v.y);
    a3 += w * bf2f_hi(v.y);
  }
  const float ss = block_reduce_sum(a0 * a0 + a1 * a1 + a2 * a2 + a3 * a3, red);
  const float rstd = 1.0f / sqrtf(ss * (1.0f / kHeadDim) + eps);
  const uint2 g = *reinterpret_cast<const uint2*>(gamma + tid * 4);
  float y0 = a0 * rstd * bf2f_lo(g.x), y1 = a1 * rstd * bf2f_hi(g.x);
  float y2 = a2 * rstd * bf2f_lo(g.y), y3 = a3 * rstd * bf2f_hi(g.y);
  const int d0 = tid * 4;
  if (d0 >= kRopeStart) {
    const double pos = (double)((i + 1) * m - 1 + rope_offset);
    float c, s;
    rope_cs(pos, (d0 - kRopeStart) / 2, theta, &c, &s);
    const float r0 = y0 * c - y1 * s, r1 = y0 * s + y1 * c;
    rope_cs(pos, (d0 - kRopeStart) / 2 + 1, theta, &c, &s);
    const float r2 = y2 * c - y3 * s, r3 = y2 * s + y3 * c;
    y0 = r0; y1 = r1; y2 = r2; y3 = r3;
  }
  const int64_t row = ring_cap > 0 ? (i % ring_cap) : i;
  uint2 o;
  o.x = pack_bf2(y0, y1);
  o.y = pack_bf2(y2, y3);
  *reinterpret_cast<uint2*>(kv_out + ((int64_t)b * kv_ld + row) * kHeadDim + d0) = o;

  if (ik_tok == nullptr) return;
  // ---- indexer key: pooled with its own logits, no norm, no RoPE ----
  pool_weights(ik_score + (int64_t)b * T, lo, hi, tok0, wt, red);
  float e = 0.f;
  if (tid < dI) {
    const uint16_t* kb = ik_tok + ((int64_t)b * T + (lo - tok0)) * dI + tid;
    for (int j = 0; j < n; ++j) e += wt[j] * bf2f(kb[(int64_t)j * dI]);
  }
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
             a.gamma, a.eps, a.theta, a.rope_offset, a.kv_out, a.kv_ld, a.ring_cap, a.ik_out,
             a.ik_scale, a.ik_ld, a.ik_fp8);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
