// Grouped output projection (page 1, "hybrid attention", CSA step 4: with c = 512 a direct
// projection of all heads is expensive, so the n_h heads are split into g groups, each group is
// projected to an intermediate width d_g, and the concatenation is projected back to d).
//
//   z[:, j*d_g:(j+1)*d_g] = o[:, heads of group j] . W_g[j]^T     (z rounded to bf16)
//   y = z . W_o^T  (+ the residual stream, optionally)
//
// The same weight-streaming kernel also serves the input projections of a layer (one pass over
// the concatenated projection weights from the hidden state, outputs scattered to their consumers).
//
// Both stages are Y[M, N] = X[M, xoff(n) + 0..K) . W[N, K]^T with output-major weights.  At decode
// M is the batch (<= 16): the kernel streams W once from HBM straight into MFMA A-fragments
// (16 B per lane, rows contiguous), X fragments come from L2, the waves of a workgroup split K
// and are summed through LDS.  One workgroup per 16 output features; its 8 waves split K.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kUnroll = 16;
constexpr int kWaves = 8;                 // waves per workgroup, splitting K
typedef unsigned int u32x4v __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4v GU32x4v;   // global address space: global_load

__global__ void __launch_bounds__(kWaves * 64)
rowblock_gemm_kernel(const uint16_t* __restrict__ X, int64_t x_ld, const uint16_t* __restrict__ W,
                     uint16_t* Y, int64_t y_ld, int M, int N, int K, int n_per_group, const uint16_t* R,
                     int64_t r_ld) {
  __shared__ float4 red[kWaves][kWave];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int64_t xoff = (int64_t)(n0 / n_per_group) * K;
  const int ksteps = K / 32;
  const int per_wave = (ksteps + kWaves - 1) / kWaves;
  const int ks0 = w * per_wave;
  int ks1 = ks0 + per_wave;
  if (ks1 > ksteps) ks1 = ksteps;
  const uint16_t* wrow = W + (int64_t)(n0 + c16) * K + 8 * g;

  for (int m0 = 0; m0 < M; m0 += 16) {
    const int mrow = m0 + c16;
    const bool mv = mrow < M;
    const uint16_t* xrow = X + (int64_t)(mv ? mrow : M - 1) * x_ld + xoff + 8 * g;
    floatx4 acc = {0.f, 0.f, 0.f, 0.f};
    int ks = ks0;
    for (; ks + kUnroll <= ks1; ks += kUnroll) {
      uint4 wa[kUnroll], xb[kUnroll];
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) {
        wa[u] = *reinterpret_cast<const uint4*>(wrow + 32 * (ks + u));
        const uint4 xv = *reinterpret_cast<const uint4*>(xrow + 32 * (ks + u));
        xb[u] = mv ? xv : make_uint4(0, 0, 0, 0);
      }
#pragma unroll
      for (int u = 0; u < kUnroll; ++u) acc = mfma_bf16(wa[u], xb[u], acc);
    }
    for (; ks < ks1; ++ks) {
      const uint4 wa = *reinterpret_cast<const uint4*>(wrow + 32 * ks);
      const uint4 xv = *reinterpret_cast<const uint4*>(xrow + 32 * ks);
      const uint4 xb = mv ? xv : make_uint4(0, 0, 0, 0);
      acc = mfma_bf16(wa, xb, acc);
    }
    // acc: lane holds column m0 + c16, rows n0 + 4g .. +3
    red[w][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
    __syncthreads();
    if (w == 0) {
      float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
      for (int v = 0; v < kWaves; ++v) {
        const float4 a = red[v][lane];
        y0 += a.x; y1 += a.y; y2 += a.z; y3 += a.w;
      }
      if (mv) {
        if (R != nullptr) {
          const uint2 rv = *reinterpret_cast<const uint2*>(R + (int64_t)mrow * r_ld + n0 + 4 * g);
          y0 += bf2f_lo(rv.x); y1 += bf2f_hi(rv.x); y2 += bf2f_lo(rv.y); y3 += bf2f_hi(rv.y);
        }
        uint2 o;
        o.x = pack_bf2(y0, y1);
        o.y = pack_bf2(y2, y3);
        *reinterpret_cast<uint2*>(Y + (int64_t)mrow * y_ld + n0 + 4 * g) = o;
      }
    }
    __syncthreads();
  }
}

// Decode shapes (M <= 8, K = 4096 or 8192): the workgroup's slice of X (M x K) is staged once in
// LDS, and each wave issues all of its W loads (KS k-steps of 16 B per lane) before the first MFMA,
// so a CU has its whole share of the weights in flight.  X rows >= M are zero in the B fragments.
//
// Epilogue options: R adds a residual (Y = X . W^T + R, summed in fp32); SEG scatters the output
// columns into the segments of a ProjSegments table (each segment its own destination, row stride and
// bf16 / fp32 type), so one pass over a concatenated weight matrix feeds several consumers.
template <int K, bool SEG>
__global__ void __launch_bounds__(kWaves * 64)
rowblock_gemv_kernel(const uint16_t* __restrict__ X, int64_t x_ld, const uint16_t* __restrict__ W,
                     uint16_t* Y, int64_t y_ld, int M, int n_per_group, const uint16_t* R, int64_t r_ld,
                     ProjSegments seg) {
  constexpr int KS = K / 32 / kWaves;      // k-steps per wave
  constexpr int kXStride = K + 8;          // bf16 per staged X row (16 B pad)
  __shared__ __align__(16) uint16_t sx[8 * kXStride];
  __shared__ float4 red[kWaves][kWave];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int n0 = blockIdx.x * 16;
  const int64_t xoff = (int64_t)(n0 / n_per_group) * K;

  // all of this wave's W fragments in flight (rows n0 + c16, k-steps w*KS ..)
  const GU32x4v* wp = reinterpret_cast<const GU32x4v*>(reinterpret_cast<uintptr_t>(
      W + (int64_t)(n0 + c16) * K + 32 * (w * KS) + 8 * g));
  uint4 wa[KS];
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const u32x4v x = wp[4 * u];
    wa[u] = make_uint4(x.x, x.y, x.z, x.w);
  }
  // X slice -> LDS (rows >= M are never read)
  constexpr int kChunks = 8 * K / 8;       // 16 B chunks of the 8-row slice
#pragma unroll
  for (int u = 0; u < kChunks / (kWaves * 64); ++u) {
    const int i = threadIdx.x + u * kWaves * 64;
    const int m = i / (K / 8), kc = i % (K / 8);
    const int ms = m < M ? m : M - 1;                  // always a readable row
    const uint4 x = *reinterpret_cast<const uint4*>(X + (int64_t)ms * x_ld + xoff + 8 * kc);
    *reinterpret_cast<uint4*>(&sx[m * kXStride + 8 * kc]) = x;
  }
  __syncthreads();
  floatx4 acc = {0.f, 0.f, 0.f, 0.f};
  const bool mv = c16 < M;
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const uint4 xv = *reinterpret_cast<const uint4*>(&sx[(mv ? c16 : 0) * kXStride + 32 * (w * KS + u) + 8 * g]);
    acc = mfma_bf16(wa[u], mv ? xv : make_uint4(0, 0, 0, 0), acc);
  }
  // acc: lane holds column (m) c16, rows n0 + 4g .. +3; sum the 8 waves' K slices
  red[w][lane] = make_float4(acc[0], acc[1], acc[2], acc[3]);
  __syncthreads();
  if (w == 0) {
    float y0 = 0.f, y1 = 0.f, y2 = 0.f, y3 = 0.f;
#pragma unroll
    for (int v = 0; v < kWaves; ++v) {
      const float4 a = red[v][lane];
      y0 += a.x; y1 += a.y; y2 += a.z; y3 += a.w;
    }
    if (mv && R != nullptr) {
      const uint2 rv = *reinterpret_cast<const uint2*>(R + (int64_t)c16 * r_ld + n0 + 4 * g);
      y0 += bf2f_lo(rv.x); y1 += bf2f_hi(rv.x); y2 += bf2f_lo(rv.y); y3 += bf2f_hi(rv.y);
    }
    if (mv && !SEG) {
      uint2 o;
      o.x = pack_bf2(y0, y1);
      o.y = pack_bf2(y2, y3);
      *reinterpret_cast<uint2*>(Y + (int64_t)c16 * y_ld + n0 + 4 * g) = o;
    } else if (mv) {
      const float yv[4] = {y0, y1, y2, y3};
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int n = n0 + 4 * g + i;
        int sidx = 0;
        while (sidx < seg.n && n >= seg.end[sidx]) ++sidx;
        if (sidx == seg.n) continue;                  // padding rows of W
        const int64_t col = n - (sidx ? seg.end[sidx - 1] : 0);
        const int64_t at = (int64_t)c16 * seg.ld[sidx] + col;
        if (seg.f32[sidx]) static_cast<float*>(seg.dst[sidx])[at] = yv[i];
        else static_cast<uint16_t*>(seg.dst[sidx])[at] = (uint16_t)f2bf(yv[i]);
      }
    }
  }
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Y = X . W^T for one stage: the staged-X kernel at the decode shapes, else the general one.
void launch_stage(const char* name, const uint16_t* X, int64_t x_ld, const uint16_t* W, uint16_t* Y, int64_t y_ld,
                  int M, int N, int K, int n_per_group, hipStream_t st, const uint16_t* R = nullptr,
                  int64_t r_ld = 0) {
  const ProjSegments none{};
  if (M <= 8 && K == 4096) {
    LCS_LAUNCH(name, (rowblock_gemv_kernel<4096, false>), dim3((unsigned)(N / 16)), dim3(kWaves * 64), 0, st, X, x_ld,
               W, Y, y_ld, M, n_per_group, R, r_ld, none);
  } else if (M <= 8 && K == 8192) {
    LCS_LAUNCH(name, (rowblock_gemv_kernel<8192, false>), dim3((unsigned)(N / 16)), dim3(kWaves * 64), 0, st, X, x_ld,
               W, Y, y_ld, M, n_per_group, R, r_ld, none);
  } else {
    LCS_LAUNCH(name, rowblock_gemm_kernel, dim3((unsigned)(N / 16)), dim3(kWaves * 64), 0, st, X, x_ld, W, Y, y_ld,
               M, N, K, n_per_group, R, r_ld);
  }
}

}  // namespace

size_t out_proj_workspace(int M, int g, int d_g) { return al256((size_t)M * g * d_g * 2); }

int launch_out_proj(const OutProjArgs& a, hipStream_t st) {
  uint16_t* z = static_cast<uint16_t*>(a.ws);
  const int kg = a.H / a.g * a.c;
  const int nz = a.g * a.d_g;
  launch_stage("out_proj_group_kernel", a.o, (int64_t)a.H * a.c, a.w_g, z, (int64_t)nz, a.M, nz, kg, a.d_g, st);
  launch_stage("out_proj_out_kernel", z, (int64_t)nz, a.w_o, a.y, (int64_t)a.d, a.M, a.d, nz, a.d, st, a.resid,
               (int64_t)a.d);
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

int launch_input_proj(const uint16_t* h, int M, int d, const uint16_t* w, int n_rows, const ProjSegments& seg,
                      hipStream_t st) {
  if (d == 4096) {
    LCS_LAUNCH("input_proj_kernel", (rowblock_gemv_kernel<4096, true>), dim3((unsigned)(n_rows / 16)),
               dim3(kWaves * 64), 0, st, h, (int64_t)d, w, nullptr, 0, M, n_rows, nullptr, 0, seg);
  } else {
    LCS_LAUNCH("input_proj_kernel", (rowblock_gemv_kernel<8192, true>), dim3((unsigned)(n_rows / 16)),
               dim3(kWaves * 64), 0, st, h, (int64_t)d, w, nullptr, 0, M, n_rows, nullptr, 0, seg);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
