// Grouped output projection (page 1, "hybrid attention", CSA step 4: with c = 512 a direct
// projection of all heads is expensive, so the n_h heads are split into g groups, each group is
// projected to an intermediate width d_g, and the concatenation is projected back to d).
//
//   z[:, j*d_g:(j+1)*d_g] = o[:, heads of group j] . W_g[j]^T     (z rounded to bf16)
//   y = z . W_o^T
//
// Both stages are Y[M, N] = X[M, xoff(n) + 0..K) . W[N, K]^T with output-major weights.  At decode
// M is the batch (<= 16): the kernel streams W once from HBM straight into MFMA A-fragments
// (16 B per lane, rows contiguous), X fragments come from L2, the 4 waves of a workgroup split K
// and are summed through LDS.  One workgroup per 16 output features.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kUnroll = 8;

__global__ void __launch_bounds__(256)
rowblock_gemm_kernel(const uint16_t* __restrict__ X, int64_t x_ld, const uint16_t* __restrict__ W,
                     uint16_t* __restrict__ Y, int64_t y_ld, int M, int N, int K, int n_per_group) {
  __shared__ float4 red[4][kWave];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int64_t xoff = (int64_t)(n0 / n_per_group) * K;
  const int ksteps = K / 32;
  const int per_wave = (ksteps + 3) / 4;
  const int ks0 = w * per_wave;
  int ks1 = ks0 + per_wave;
  if (ks1 > ksteps) ks1 = ksteps;
  const uint16_t* wrow = W + (int64_t)(n0 + c16) * K + 8 * g;

  for (int m0 = 0; m0 < M; m0 += 16) {
    const int mrow = m0 + c16;
    const bool mv = mrow < M;
    const uint16_t* xrow = X + (int64_t)(mv ? mrow : 0) * x_ld + xoff + 8 * g;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int ks = ks0;
    for (; ks + kUnroll <= ks1; ks += kUnroll) {
      uint4 wa[kUnroll], xb[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        wa[u] = *reinterpret_cast<const uint4*>(wrow + 32 * (ks + u));
        xb[u] = mv ? *reinterpret_cast<const uint4*>(xrow + 32 * (ks + u)) : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc = mfma_bf16(wa[u], xb[u], acc);
    }
    for (; ks < ks1; ++ks) {
      const uint4 wa = *reinterpret_cast<const uint4*>(wrow + 32 * ks);
      const uint4 xb = mv ? *reinterpret_cast<const uint4*>(xrow + 32 * ks) : make_uint4(0, 0, 0, 0);
      acc = mfma_bf16(wa, xb, acc);
    }
    // acc: lane holds column m0 + c16, rows n0 + 4g .. +3
    red[w][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (w == 0) {
      const float4 a0 = red[0][lane], a1 = red[1][lane], a2 = red[2][lane], a3 = red[3][lane];
      const float y0 = (a0.x + a1.x) + (a2.x + a3.x);
      const float y1 = (a0.y + a1.y) + (a2.y + a3.y);
      const float y2 = (a0.z + a1.z) + (a2.z + a3.z);
      const float y3 = (a0.w + a1.w) + (a2.w + a3.w);
      if (mv) {
        uint2 o;
        o.x = pack_bf2(y0, y1);
        o.y = pack_bf2(y2, y3);
        *reinterpret_cast<uint2*>(Y + (int64_t)mrow * y_ld + n0 + 4 * g) = o;
      }
    }
    __syncthreads();
  }
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

}  // namespace

size_t out_proj_workspace(int M, int g, int d_g) { return al256((size_t)M * g * d_g * 2); }

int launch_out_proj(const OutProjArgs& a, hipStream_t st) {
  uint16_t* z = static_cast<uint16_t*>(a.ws);
  const int kg = a.H / a.g * a.c;
  const int nz = a.g * a.d_g;
  LCS_LAUNCH("out_proj_group_kernel", rowblock_gemm_kernel, dim3((unsigned)(nz / 16)), dim3(256), 0, st,
             a.o, (int64_t)a.H * a.c, a.w_g, z, (int64_t)nz, a.M, nz, kg, a.d_g);
  LCS_LAUNCH("out_proj_out_kernel", rowblock_gemm_kernel, dim3((unsigned)(a.d / 16)), dim3(256), 0, st,
             z, (int64_t)nz, a.w_o, a.y, (int64_t)a.d, a.M, a.d, nz, a.d);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
