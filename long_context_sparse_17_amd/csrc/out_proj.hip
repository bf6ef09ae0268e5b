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
#include <mutex>

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

  // the X slice's loads first (L2 hits; rows >= M are never read), then all of this wave's W
  // fragments (rows n0 + c16, k-steps w*KS ..): loads return in order, so X is staged while W streams
  constexpr int kChunks = 8 * K / 8;       // 16 B chunks of the 8-row slice
  constexpr int kXPer = kChunks / (kWaves * 64);
  uint4 xs[kXPer];
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int i = threadIdx.x + u * kWaves * 64;
    const int m = i / (K / 8), kc = i % (K / 8);
    const int ms = m < M ? m : M - 1;                  // always a readable row
    xs[u] = *reinterpret_cast<const uint4*>(X + (int64_t)ms * x_ld + xoff + 8 * kc);
  }
  const GU32x4v* wp = reinterpret_cast<const GU32x4v*>(reinterpret_cast<uintptr_t>(
      W + (int64_t)(n0 + c16) * K + 32 * (w * KS) + 8 * g));
  uint4 wa[KS];
#pragma unroll
  for (int u = 0; u < KS; ++u) {
    const u32x4v x = wp[4 * u];
    wa[u] = make_uint4(x.x, x.y, x.z, x.w);
  }
#pragma unroll
  for (int u = 0; u < kXPer; ++u) {
    const int i = threadIdx.x + u * kWaves * 64;
    const int m = i / (K / 8), kc = i % (K / 8);
    *reinterpret_cast<uint4*>(&sx[m * kXStride + 8 * kc]) = xs[u];
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

// Prefill shapes (M >= 64): a tiled GEMM.  A workgroup computes a 128 x 128 block of Y (output
// features n0 .., rows m0 ..), stepping through K in slices of 64: the W and X slices (128 rows x
// 128 B each) go global -> registers -> LDS, double-buffered so the next slice's loads are in flight
// while the current one feeds the matrix cores; one barrier per slice.  Four waves in a 2 x 2
// arrangement each own a 64 x 64 sub-block (4 x 4 MFMA tiles, W fragments as A, X fragments as B,
// so a lane ends with 4 consecutive features of one row).  Each W and X element is read from
// global memory once per 128-row / 128-feature block instead of once per 16 rows.
constexpr int kTgM = 128, kTgN = 128, kTgK = 64;
constexpr int kTgStride = kTgK + 8;       // bf16 per LDS row (144 B: 16 rows of a fragment read start 36 words apart)
constexpr int kTgThreads = 256;

__global__ void __launch_bounds__(kTgThreads, 2)
tile_gemm_kernel(const uint16_t* __restrict__ X, int64_t x_ld, const uint16_t* __restrict__ W, uint16_t* Y,
                 int64_t y_ld, int M, int K, int n_per_group, const uint16_t* R, int64_t r_ld) {
  __shared__ __align__(16) uint16_t sw[2][kTgN * kTgStride];
  __shared__ __align__(16) uint16_t sxm[2][kTgM * kTgStride];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int wn = w & 1, wm = w >> 1;       // this wave's 64 x 64 sub-block
  const int n0 = blockIdx.x * kTgN;
  const int m0 = blockIdx.y * kTgM;
  const int64_t xoff = (int64_t)(n0 / n_per_group) * K;

  // global -> register staging: 16 B chunks, chunk q = tid + 256 j (j = 0..3) is row q / 8, k-chunk
  // q % 8 of the slice; rows past M read row M - 1 (never stored)
  const uint16_t* wsrc[4];
  const uint16_t* xsrc[4];
  int lds_off[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int q = threadIdx.x + kTgThreads * j;
    const int row = q >> 3, kc = q & 7;
    const int m = m0 + row < M ? m0 + row : M - 1;
    wsrc[j] = W + (int64_t)(n0 + row) * K + 8 * kc;
    xsrc[j] = X + (int64_t)m * x_ld + xoff + 8 * kc;
    lds_off[j] = row * kTgStride + 8 * kc;
  }
  floatx4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  const int nk = K / kTgK;
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    *reinterpret_cast<uint4*>(&sw[0][lds_off[j]]) = *reinterpret_cast<const uint4*>(wsrc[j]);
    *reinterpret_cast<uint4*>(&sxm[0][lds_off[j]]) = *reinterpret_cast<const uint4*>(xsrc[j]);
  }
  __syncthreads();
  // one 64-deep slice from LDS slot `slot` into the accumulators
  auto multiply = [&](int slot) {
#pragma unroll
    for (int ks = 0; ks < kTgK / 32; ++ks) {
      uint4 fa[4], fb[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)                     // W rows (features) wn*64 + 16i + c16
        fa[i] = *reinterpret_cast<const uint4*>(&sw[slot][(wn * 64 + 16 * i + c16) * kTgStride + 32 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < 4; ++j)                     // X rows wm*64 + 16j + c16
        fb[j] = *reinterpret_cast<const uint4*>(&sxm[slot][(wm * 64 + 16 * j + c16) * kTgStride + 32 * ks + 8 * g]);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = mfma_bf16(fa[i], fb[j], acc[i][j]);
    }
  };
  for (int t = 0; t + 1 < nk; ++t) {
    const int slot = t & 1;
    const int k0 = (t + 1) * kTgK;                  // slice t + 1 in flight while slice t is multiplied
    uint4 nw0 = *reinterpret_cast<const uint4*>(wsrc[0] + k0), nx0 = *reinterpret_cast<const uint4*>(xsrc[0] + k0);
    uint4 nw1 = *reinterpret_cast<const uint4*>(wsrc[1] + k0), nx1 = *reinterpret_cast<const uint4*>(xsrc[1] + k0);
    uint4 nw2 = *reinterpret_cast<const uint4*>(wsrc[2] + k0), nx2 = *reinterpret_cast<const uint4*>(xsrc[2] + k0);
    uint4 nw3 = *reinterpret_cast<const uint4*>(wsrc[3] + k0), nx3 = *reinterpret_cast<const uint4*>(xsrc[3] + k0);
    multiply(slot);
    // the other slot was last read before the previous barrier
    uint16_t* dw = sw[slot ^ 1];
    uint16_t* dx = sxm[slot ^ 1];
    *reinterpret_cast<uint4*>(&dw[lds_off[0]]) = nw0; *reinterpret_cast<uint4*>(&dx[lds_off[0]]) = nx0;
    *reinterpret_cast<uint4*>(&dw[lds_off[1]]) = nw1; *reinterpret_cast<uint4*>(&dx[lds_off[1]]) = nx1;
    *reinterpret_cast<uint4*>(&dw[lds_off[2]]) = nw2; *reinterpret_cast<uint4*>(&dx[lds_off[2]]) = nx2;
    *reinterpret_cast<uint4*>(&dw[lds_off[3]]) = nw3; *reinterpret_cast<uint4*>(&dx[lds_off[3]]) = nx3;
    __syncthreads();
  }
  multiply((nk - 1) & 1);

  // acc[i][j]: lane holds row m0 + wm*64 + 16j + c16, features n0 + wn*64 + 16i + 4g .. +3
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = m0 + wm * 64 + 16 * j + c16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + 16 * i + 4 * g;
      float y0 = acc[i][j][0], y1 = acc[i][j][1], y2 = acc[i][j][2], y3 = acc[i][j][3];
      if (R != nullptr) {
        const uint2 rv = *reinterpret_cast<const uint2*>(R + (int64_t)m * r_ld + n);
        y0 += bf2f_lo(rv.x); y1 += bf2f_hi(rv.x); y2 += bf2f_lo(rv.y); y3 += bf2f_hi(rv.y);
      }
      *reinterpret_cast<uint2*>(Y + (int64_t)m * y_ld + n) = make_uint2(pack_bf2(y0, y1), pack_bf2(y2, y3));
    }
  }
}

// Large prefill shapes (M >= 512): 256 x 256 blocks, one workgroup of 8 waves per CU (two per SIMD),
// each wave owning 128 rows x 64 features (4 x 8 MFMA tiles, 128 accumulators).  A wave reads 0.375
// KiB of fragments from LDS per MFMA instead of 0.5 (128 x 128 blocks of 64 x 64 waves).  Same slice
// pipeline as tile_gemm_kernel: K in slices of 64 through double-buffered LDS (global -> registers ->
// LDS, rows 144 B apart), one barrier per slice.
constexpr int kTg2 = 256;                  // block rows and features
constexpr int kTg2Threads = 512;
constexpr int kTg2Chunks = kTg2 * kTgK / 8 / kTg2Threads;   // 16 B chunks per thread per operand slice (4)

__global__ void __launch_bounds__(kTg2Threads, 1)
tile_gemm256_kernel(const uint16_t* __restrict__ X, int64_t x_ld, const uint16_t* __restrict__ W, uint16_t* Y,
                    int64_t y_ld, int M, int K, int n_per_group, const uint16_t* R, int64_t r_ld) {
  __shared__ __align__(16) uint16_t sw[2][kTg2 * kTgStride];
  __shared__ __align__(16) uint16_t sxm[2][kTg2 * kTgStride];
  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int wn = w & 3, wm = w >> 2;       // this wave's features n0 + 64 wn .., rows m0 + 128 wm ..
  const int n0 = blockIdx.x * kTg2;
  const int m0 = blockIdx.y * kTg2;
  const int64_t xoff = (int64_t)(n0 / n_per_group) * K;

  // global -> register staging: chunk q = tid + 512 j is row q / 8, k-chunk q % 8 of the slice; rows
  // past M read row M - 1 (never stored)
  const int kc = threadIdx.x & 7, row0 = threadIdx.x >> 3;   // rows row0 + 64 j
  const uint16_t* wbase = W + (int64_t)(n0 + row0) * K + 8 * kc;
  const uint16_t* xbase = X + xoff + 8 * kc;
  const bool xfull = m0 + kTg2 <= M;                          // uniform: every block row exists
  const int lds0 = row0 * kTgStride + 8 * kc;                // + 64 j rows
  floatx4 acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 8; ++j) acc[i][j] = floatx4{0.f, 0.f, 0.f, 0.f};

  static_assert(kTg2Chunks == 4, "four staging chunks per operand");
  // X row offsets of the thread's 4 chunks (rows past M: row M - 1)
  int64_t xr[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int m = xfull || m0 + row0 + 64 * j < M ? m0 + row0 + 64 * j : M - 1;
    xr[j] = (int64_t)m * x_ld;
  }
  const int64_t wr = (int64_t)64 * K;
#define LCS_TG2_FETCH(k0)                                                             \
  const uint4 nw0 = *reinterpret_cast<const uint4*>(wbase + (k0));                    \
  const uint4 nw1 = *reinterpret_cast<const uint4*>(wbase + wr + (k0));               \
  const uint4 nw2 = *reinterpret_cast<const uint4*>(wbase + 2 * wr + (k0));           \
  const uint4 nw3 = *reinterpret_cast<const uint4*>(wbase + 3 * wr + (k0));           \
  const uint4 nx0 = *reinterpret_cast<const uint4*>(xbase + xr[0] + (k0));            \
  const uint4 nx1 = *reinterpret_cast<const uint4*>(xbase + xr[1] + (k0));            \
  const uint4 nx2 = *reinterpret_cast<const uint4*>(xbase + xr[2] + (k0));            \
  const uint4 nx3 = *reinterpret_cast<const uint4*>(xbase + xr[3] + (k0));
#define LCS_TG2_COMMIT(slot)                                                          \
  *reinterpret_cast<uint4*>(&sw[slot][lds0]) = nw0;                                   \
  *reinterpret_cast<uint4*>(&sw[slot][lds0 + 64 * kTgStride]) = nw1;                  \
  *reinterpret_cast<uint4*>(&sw[slot][lds0 + 128 * kTgStride]) = nw2;                 \
  *reinterpret_cast<uint4*>(&sw[slot][lds0 + 192 * kTgStride]) = nw3;                 \
  *reinterpret_cast<uint4*>(&sxm[slot][lds0]) = nx0;                                  \
  *reinterpret_cast<uint4*>(&sxm[slot][lds0 + 64 * kTgStride]) = nx1;                 \
  *reinterpret_cast<uint4*>(&sxm[slot][lds0 + 128 * kTgStride]) = nx2;                \
  *reinterpret_cast<uint4*>(&sxm[slot][lds0 + 192 * kTgStride]) = nx3;
  // one 64-deep slice: per 32-deep step, the wave's 4 W fragments, then each X fragment against all 4
  auto multiply = [&](int slot) {
#pragma unroll
    for (int ks = 0; ks < kTgK / 32; ++ks) {
      uint4 fa[4];
#pragma unroll
      for (int i = 0; i < 4; ++i)                     // W rows (features) wn*64 + 16i + c16
        fa[i] = *reinterpret_cast<const uint4*>(&sw[slot][(wn * 64 + 16 * i + c16) * kTgStride + 32 * ks + 8 * g]);
#pragma unroll
      for (int j = 0; j < 8; ++j) {                   // X rows wm*128 + 16j + c16
        const uint4 fb = *reinterpret_cast<const uint4*>(&sxm[slot][(wm * 128 + 16 * j + c16) * kTgStride + 32 * ks + 8 * g]);
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i][j] = mfma_bf16(fa[i], fb, acc[i][j]);
      }
    }
  };
  const int nk = K / kTgK;
  {
    LCS_TG2_FETCH(0)
    LCS_TG2_COMMIT(0)
  }
  __syncthreads();
  for (int t = 0; t + 1 < nk; ++t) {
    LCS_TG2_FETCH((t + 1) * kTgK)                     // slice t + 1 in flight while slice t is multiplied
    multiply(t & 1);
    LCS_TG2_COMMIT((t + 1) & 1)                       // that slot was last read before the previous barrier
    __syncthreads();
  }
  multiply((nk - 1) & 1);
#undef LCS_TG2_FETCH
#undef LCS_TG2_COMMIT

  // acc[i][j]: lane holds row m0 + wm*128 + 16j + c16, features n0 + wn*64 + 16i + 4g .. +3
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int m = m0 + wm * 128 + 16 * j + c16;
    if (m >= M) continue;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int n = n0 + wn * 64 + 16 * i + 4 * g;
      float y0 = acc[i][j][0], y1 = acc[i][j][1], y2 = acc[i][j][2], y3 = acc[i][j][3];
      if (R != nullptr) {
        const uint2 rv = *reinterpret_cast<const uint2*>(R + (int64_t)m * r_ld + n);
        y0 += bf2f_lo(rv.x); y1 += bf2f_hi(rv.x); y2 += bf2f_lo(rv.y); y3 += bf2f_hi(rv.y);
      }
      *reinterpret_cast<uint2*>(Y + (int64_t)m * y_ld + n) = make_uint2(pack_bf2(y0, y1), pack_bf2(y2, y3));
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
  } else if (M >= 512 && N % kTg2 == 0 && n_per_group % kTg2 == 0 && K % kTgK == 0) {
    LCS_LAUNCH(name, tile_gemm256_kernel, dim3((unsigned)(N / kTg2), (unsigned)((M + kTg2 - 1) / kTg2)),
               dim3(kTg2Threads), 0, st, X, x_ld, W, Y, y_ld, M, K, n_per_group, R, r_ld);
  } else if (M >= 64 && N % kTgN == 0 && n_per_group % kTgN == 0 && K % kTgK == 0) {
    LCS_LAUNCH(name, tile_gemm_kernel, dim3((unsigned)(N / kTgN), (unsigned)((M + kTgM - 1) / kTgM)), dim3(kTgThreads),
               0, st, X, x_ld, W, Y, y_ld, M, K, n_per_group, R, r_ld);
  } else {
    LCS_LAUNCH(name, rowblock_gemm_kernel, dim3((unsigned)(N / 16)), dim3(kWaves * 64), 0, st, X, x_ld, W, Y, y_ld,
               M, N, K, n_per_group, R, r_ld);
  }
}

}  // namespace

size_t out_proj_workspace(int M, int g, int d_g) { return al256((size_t)M * g * d_g * 2); }

}  // namespace lcs

// Scratch of the allocation-free grouped projection: the intermediate z lives in this file-scope
// device array instead of a caller workspace.  Each GPU the library runs on holds its own copy
// until the process ends; every call on one GPU shares it, so calls that overlap on one GPU race.
// z is written in full before it is read, so nothing needs clearing between calls.
static __device__ __align__(256) uint8_t scratch[lcs::kOutProjScratchBytes];

namespace lcs {

// Device address of `scratch` on the current device, looked up once per device with that device
// current (the host-side name is only a stand-in, never a device address).
int out_proj_scratch(void** ptr) {
  constexpr int kMaxDevices = 64;
  static std::mutex mu;
  static void* dev_ptr[kMaxDevices] = {};
  int dev = -1;
  if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return 4;
  std::lock_guard<std::mutex> lk(mu);
  if (dev_ptr[dev] == nullptr) {
    void* p = nullptr;
    if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || p == nullptr) return 4;
    dev_ptr[dev] = p;
  }
  *ptr = dev_ptr[dev];
  return 0;
}

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
