// mHC: mixing of the n residual streams between layers (page 1, section on mHC: the streams are
// mixed by a matrix B held on the doubly stochastic matrices by Sinkhorn-Knopp, alternating row
// and column normalisation for 20 rounds per layer, with the input map A and output map C passed
// through a sigmoid; page 4 section 3.2).
//
// Per token: B = Sinkhorn-Knopp(exp(mixing logits)), C = sigmoid(C~), A = sigmoid(A~ of the next
// layer); the streams update as X'_i = sum_j B_ij X_j + C_i y and the next layer's input is
// h = sum_i A_i X'_i.  The n x n projection is tiny (n <= 8) and sequential: one lane per token
// runs all its rounds in registers (exp of the row-max-shifted logits, which the first row
// normalisation makes exact), then the workgroup streams the token's n rows of d bf16 values,
// 16 bytes per thread per row, and writes X' (bf16) and h (bf16, from the fp32 X').  Each thread
// reads a chunk of every stream before writing it back, so X' may overwrite X in place.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kThreads = 256;
constexpr int kTokPerWG = 4;              // tokens per workgroup (their projections run in parallel lanes)

// Sinkhorn-Knopp rounds of one n x n matrix of logits, in place: M <- exp(L - rowmax), then `iters`
// rounds of (rows / row sums, columns / column sums).
template <int N>
__device__ __forceinline__ void sinkhorn_rounds(float (&M)[N][N], int iters) {
#pragma unroll
  for (int i = 0; i < N; ++i) {
    float mx = M[i][0];
#pragma unroll
    for (int j = 1; j < N; ++j) mx = fmaxf(mx, M[i][j]);
#pragma unroll
    for (int j = 0; j < N; ++j) M[i][j] = __expf(M[i][j] - mx);
  }
  for (int r = 0; r < iters; ++r) {
#pragma unroll
    for (int i = 0; i < N; ++i) {
      float s = 0.f;
#pragma unroll
      for (int j = 0; j < N; ++j) s += M[i][j];
      const float inv = 1.0f / s;
#pragma unroll
      for (int j = 0; j < N; ++j) M[i][j] *= inv;
    }
#pragma unroll
    for (int j = 0; j < N; ++j) {
      float s = 0.f;
#pragma unroll
      for (int i = 0; i < N; ++i) s += M[i][j];
      const float inv = 1.0f / s;
#pragma unroll
      for (int i = 0; i < N; ++i) M[i][j] *= inv;
    }
  }
}

__device__ __forceinline__ float sigmoid(float x) { return 1.0f / (1.0f + __expf(-x)); }

template <int N>
__global__ void __launch_bounds__(kThreads)
sinkhorn_kernel(const float* __restrict__ logits, int T, int iters, float* __restrict__ out) {
  const int t = blockIdx.x * kThreads + threadIdx.x;
  if (t >= T) return;
  float M[N][N];
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) M[i][j] = logits[(int64_t)t * N * N + i * N + j];
  sinkhorn_rounds<N>(M, iters);
#pragma unroll
  for (int i = 0; i < N; ++i)
#pragma unroll
    for (int j = 0; j < N; ++j) out[(int64_t)t * N * N + i * N + j] = M[i][j];
}

template <int N>
__global__ void __launch_bounds__(kThreads)
mhc_mix_kernel(const uint16_t* x, const uint16_t* __restrict__ y, const float* __restrict__ logits,
               int T, int d, int iters, uint16_t* x_out, uint16_t* __restrict__ h_out) {
  constexpr int kCoef = N * N + 2 * N;    // B (row-major), C, A
  __shared__ float coef[kTokPerWG][kCoef];
  const int tok0 = blockIdx.x * kTokPerWG;
  if (threadIdx.x < kTokPerWG && tok0 + (int)threadIdx.x < T) {
    const float* L = logits + (int64_t)(tok0 + threadIdx.x) * kCoef;
    float M[N][N];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) M[i][j] = L[i * N + j];
    float cz[2 * N];
#pragma unroll
    for (int k = 0; k < 2 * N; ++k) cz[k] = L[N * N + k];
    sinkhorn_rounds<N>(M, iters);
    float* c = coef[threadIdx.x];
#pragma unroll
    for (int i = 0; i < N; ++i)
#pragma unroll
      for (int j = 0; j < N; ++j) c[i * N + j] = M[i][j];
#pragma unroll
    for (int k = 0; k < 2 * N; ++k) c[N * N + k] = sigmoid(cz[k]);
  }
  __syncthreads();

  for (int tt = 0; tt < kTokPerWG; ++tt) {
    const int tok = tok0 + tt;
    if (tok >= T) break;                  // uniform
    const float* c = coef[tt];
    const uint16_t* xs = x + (int64_t)tok * N * d;
    uint16_t* xo = x_out + (int64_t)tok * N * d;
    for (int e = 8 * threadIdx.x; e < d; e += 8 * kThreads) {
      float v[N][8];
#pragma unroll
      for (int j = 0; j < N; ++j) {
        const uint4 r = *reinterpret_cast<const uint4*>(xs + (int64_t)j * d + e);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { v[j][2 * q] = bf2f_lo(w[q]); v[j][2 * q + 1] = bf2f_hi(w[q]); }
      }
      float yv[8];
      {
        const uint4 r = *reinterpret_cast<const uint4*>(y + (int64_t)tok * d + e);
        const uint32_t w[4] = {r.x, r.y, r.z, r.w};
#pragma unroll
        for (int q = 0; q < 4; ++q) { yv[2 * q] = bf2f_lo(w[q]); yv[2 * q + 1] = bf2f_hi(w[q]); }
      }
      float hv[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
#pragma unroll
      for (int i = 0; i < N; ++i) {
        float o[8];
#pragma unroll
        for (int k = 0; k < 8; ++k) {
          float a = c[N * N + i] * yv[k];
#pragma unroll
          for (int j = 0; j < N; ++j) a += c[i * N + j] * v[j][k];
          o[k] = a;
        }
        uint4 pk;
        pk.x = pack_bf2(o[0], o[1]); pk.y = pack_bf2(o[2], o[3]);
        pk.z = pack_bf2(o[4], o[5]); pk.w = pack_bf2(o[6], o[7]);
        *reinterpret_cast<uint4*>(xo + (int64_t)i * d + e) = pk;
        const float ai = c[N * N + N + i];          // h from the fp32 streams: one rounding, at the end
#pragma unroll
        for (int k = 0; k < 8; ++k) hv[k] += ai * o[k];
      }
      if (h_out != nullptr) {
        uint4 pk;
        pk.x = pack_bf2(hv[0], hv[1]); pk.y = pack_bf2(hv[2], hv[3]);
        pk.z = pack_bf2(hv[4], hv[5]); pk.w = pack_bf2(hv[6], hv[7]);
        *reinterpret_cast<uint4*>(h_out + (int64_t)tok * d + e) = pk;
      }
    }
  }
}

template <int N>
int launch_mhc_n(const MhcArgs& a, hipStream_t stream) {
  if (a.x == nullptr) {
    LCS_LAUNCH("sinkhorn_kernel", sinkhorn_kernel<N>, dim3((unsigned)((a.T + kThreads - 1) / kThreads)),
               dim3(kThreads), 0, stream, a.logits, a.T, a.iters, a.b_out);
  } else {
    LCS_LAUNCH("mhc_mix_kernel", mhc_mix_kernel<N>, dim3((unsigned)((a.T + kTokPerWG - 1) / kTokPerWG)),
               dim3(kThreads), 0, stream, a.x, a.y, a.logits, a.T, a.d, a.iters, a.x_out, a.h_out);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace

int launch_mhc(const MhcArgs& a, hipStream_t stream) {
  switch (a.n) {
    case 1: return launch_mhc_n<1>(a, stream);
    case 2: return launch_mhc_n<2>(a, stream);
    case 3: return launch_mhc_n<3>(a, stream);
    case 4: return launch_mhc_n<4>(a, stream);
    case 5: return launch_mhc_n<5>(a, stream);
    case 6: return launch_mhc_n<6>(a, stream);
    case 7: return launch_mhc_n<7>(a, stream);
    case 8: return launch_mhc_n<8>(a, stream);
    default: return 2;
  }
}

}  // namespace lcs
