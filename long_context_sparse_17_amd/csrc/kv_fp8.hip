// fp8 storage of K=V rows (the pages: FP8 for the KV cache, halving its memory, page 2 on HCA's
// mixed FP4 + FP8 precision): each 512-dim row becomes E4M3FN codes with one fp32 scale
// absmax / 448, the same per-row quantiser as the indexer keys (round to nearest even, saturating).
// One wave per row, 8 dims (16 bytes) per lane.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kThreads = 256;
constexpr int kRowsPerWG = kThreads / kWave;

__global__ void __launch_bounds__(kThreads)
kv_quantize_kernel(const uint16_t* __restrict__ kv, int64_t rows, uint8_t* __restrict__ codes,
                   float* __restrict__ scales) {
  const int64_t row = (int64_t)blockIdx.x * kRowsPerWG + threadIdx.x / kWave;
  if (row >= rows) return;                 // uniform per wave
  const int lane = lane_id();
  const uint4 r = *reinterpret_cast<const uint4*>(kv + row * kHeadDim + 8 * lane);
  const uint32_t w[4] = {r.x, r.y, r.z, r.w};
  float v[8];
#pragma unroll
  for (int q = 0; q < 4; ++q) { v[2 * q] = bf2f_lo(w[q]); v[2 * q + 1] = bf2f_hi(w[q]); }
  float amax = 0.f;
#pragma unroll
  for (int k = 0; k < 8; ++k) amax = fmaxf(amax, fabsf(v[k]));
  amax = wave_max(amax);
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
  uint32_t c[2] = {0u, 0u};
#pragma unroll
  for (int k = 0; k < 8; ++k) c[k >> 2] |= f2e4m3(__fdiv_rn(v[k], sc)) << (8 * (k & 3));
  *reinterpret_cast<uint2*>(codes + row * kHeadDim + 8 * lane) = make_uint2(c[0], c[1]);
  if (lane == 0) scales[row] = sc;
}

}  // namespace

int launch_kv_quantize(const uint16_t* kv, int64_t rows, uint8_t* codes, float* scales, hipStream_t stream) {
  const int64_t grid = (rows + kRowsPerWG - 1) / kRowsPerWG;
  LCS_LAUNCH("kv_quantize_kernel", kv_quantize_kernel, dim3((unsigned)grid), dim3(kThreads), 0, stream, kv, rows,
             codes, scales);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
