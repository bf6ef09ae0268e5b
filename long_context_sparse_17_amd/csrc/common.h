// Device helpers shared by the gfx950 kernels of the hybrid compressed attention forward.
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcs {

constexpr int kHeadDim = 512;            // c (page 1, "hybrid attention", CSA step 4)
constexpr int kRopeDims = 64;            // RoPE on the last 64 dims (page 1 "Partial RoPE"; page 4 section 3.1)
constexpr int kRopeStart = kHeadDim - kRopeDims;
constexpr int kWave = 64;

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float floatx4 __attribute__((ext_vector_type(4)));
typedef int intx8 __attribute__((ext_vector_type(8)));
typedef int intx4 __attribute__((ext_vector_type(4)));

// ----------------------------------------------------------------------------------- conversions
__device__ __forceinline__ float bf2f(uint32_t b) { return __uint_as_float(b << 16); }
__device__ __forceinline__ float bf2f_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf2f_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16, round to nearest even: gfx950 converts a pair in one instruction
// (v_cvt_pk_bf16_f32); it agrees bit for bit with the rounding rule on finite values, ties and
// subnormals included, and keeps NaNs NaN.
typedef __bf16 bf16x2_hw __attribute__((ext_vector_type(2)));
typedef float floatx2_hw __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t pack_bf2(float lo, float hi) {
  return __builtin_bit_cast(uint32_t, __builtin_convertvector((floatx2_hw){lo, hi}, bf16x2_hw));
}
__device__ __forceinline__ uint32_t f2bf(float f) { return pack_bf2(f, 0.f) & 0xFFFFu; }

// fp32 -> OCP E4M3FN code: round to nearest, ties to even, saturating at +-448; -0 -> +0.
// Written from the format's definition: bias 7, 3 mantissa bits, subnormal quantum 2^-9.
__device__ __forceinline__ uint32_t f2e4m3(float v) {
  const uint32_t sign = (__float_as_uint(v) >> 24) & 0x80u;
  const float a = fminf(fabsf(v), 448.0f);
  uint32_t code;
  if (a < 0.015625f) {                           // below the smallest normal 2^-6
    code = (uint32_t)__builtin_rintf(a * 512.0f); // exact scaling, RNE to a multiple of 2^-9 (8 -> 0x08)
  } else {
    uint32_t b = __float_as_uint(a);
    b += 0x7FFFFu + ((b >> 20) & 1u);             // keep 3 mantissa bits, RNE, carry into exponent
    code = (((b >> 23) - 120u) << 3) | ((b >> 20) & 7u);
  }
  return code ? (sign | code) : 0u;
}

// Order-preserving map fp32 -> uint32 (larger float <-> larger key; +0 canonical).
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// ----------------------------------------------------------------------------------- RoPE
// Inverse frequencies theta^(-j/32) of the 32 rotated pairs, computed once on the host in fp64 and
// passed by value in the kernel arguments.
struct RopeFreq {
  double inv[kRopeDims / 2];
};

// cos/sin of pos * inv_j.  The angle is formed in fp64 (positions near 2^20 would lose their phase
// in fp32), reduced by 2*pi with a two-term Cody-Waite split (error ~1e-10 rad at 1e6 rad), and the
// reduced angle in [-pi, pi] goes to the fp32 sincos.
__device__ __forceinline__ void rope_cs(double pos, double inv_j, float* c, float* s) {
  const double phi = pos * inv_j;
  const double kq = rint(phi * 0.15915494309189535);
  double rr = fma(-kq, 6.283185307179586, phi);
  rr = fma(-kq, 2.4492935982947064e-16, rr);
  sincosf((float)rr, s, c);
}

// ----------------------------------------------------------------------------------- MFMA
// D(16x16 fp32) += A(16x32 bf16) * B(32x16 bf16).  Lane l holds A row l%16 / B column l%16 with
// the 8 k-values of group l/16; D: lane l holds column l%16, rows 4*(l/16) .. +3.
__device__ __forceinline__ floatx4 mfma_bf16(uint4 a, uint4 b, floatx4 c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}
// D(16x16 fp32) += A(16x128 e4m3) * B(128x16 e4m3), unit block scales (E8M0 127 = 2^0).
__device__ __forceinline__ floatx4 mfma_fp8(intx8 a, intx8 b, floatx4 c) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, c, 0, 0, 0, 127, 0, 127);
}
// D(16x16 fp32) = A * B with a power-of-two scale 2^(sa - 127) on each lane's 32 A values (E8M0; lane
// l holds A row l%16, k = 32 (l/16) .. +31) and unit B scales.
__device__ __forceinline__ floatx4 mfma_fp8_scale_a(intx8 a, intx8 b, int sa) {
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, floatx4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, sa, 0, 127);
}

// ----------------------------------------------------------------------------------- wave ops
// v_permlane16_swap / v_permlane32_swap (VALU, no LDS round trip): every lane receives the values
// of the lane pair (l, l ^ 16), resp. (l, l ^ 32), the lower lane's first, so combining the two
// gives the same bits in both lanes of a pair.
__device__ __forceinline__ float sum_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float sum_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return __uint_as_float(r[0]) + __uint_as_float(r[1]);
}
__device__ __forceinline__ float max_xor16(float x) {
  const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
__device__ __forceinline__ float max_xor32(float x) {
  const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(x), __float_as_uint(x), false, false);
  return fmaxf(__uint_as_float(r[0]), __uint_as_float(r[1]));
}
// Sum / max over the 4 lanes l, l ^ 16, l ^ 32, l ^ 48 (the 4 row groups of an MFMA fragment).
__device__ __forceinline__ float sum_rows4(float x) { return sum_xor32(sum_xor16(x)); }
__device__ __forceinline__ float max_rows4(float x) { return max_xor32(max_xor16(x)); }

__device__ __forceinline__ float wave_sum(float v) {
  v = sum_rows4(v);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v += __shfl_xor(v, o, kWave);
  return v;
}
__device__ __forceinline__ float wave_max(float v) {
  v = max_rows4(v);
#pragma unroll
  for (int o = 8; o >= 1; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, kWave));
  return v;
}
__device__ __forceinline__ int lane_id() { return (int)(threadIdx.x & (kWave - 1)); }

// Inclusive prefix sum over the 64 lanes of a fully active wave: DPP row_shr steps of 1, 2, 4, 8
// inside each row of 16 lanes (lanes shifted in from outside the row read 0), then the totals of
// the lower rows, read with readlane, added per row.  No LDS round trip.
__device__ __forceinline__ uint32_t wave_incl_scan(uint32_t x) {
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x111, 0xF, 0xF, false);   // row_shr:1
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x112, 0xF, 0xF, false);   // row_shr:2
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x114, 0xF, 0xF, false);   // row_shr:4
  x += (uint32_t)__builtin_amdgcn_update_dpp(0, (int)x, 0x118, 0xF, 0xF, false);   // row_shr:8
  const uint32_t t0 = (uint32_t)__builtin_amdgcn_readlane((int)x, 15);
  const uint32_t t1 = (uint32_t)__builtin_amdgcn_readlane((int)x, 31);
  const uint32_t t2 = (uint32_t)__builtin_amdgcn_readlane((int)x, 47);
  const int row = lane_id() >> 4;
  return x + (row > 0 ? t0 : 0u) + (row > 1 ? t1 : 0u) + (row > 2 ? t2 : 0u);
}

}  // namespace lcs

// ----------------------------------------------------------------------------------- host side
namespace lcs {
RopeFreq rope_freq(float theta);
// inv[j] for a per-thread j, picked with constant indices: when the table is a kernel argument these
// are scalar loads, issued at once, instead of an indexed vector load that the compiler places at its
// use, behind every vector load in flight (vector loads complete in order)
__device__ __forceinline__ double rope_inv(const RopeFreq& rf, int j) {
  double v = 0.0;
#pragma unroll
  for (int i = 0; i < kRopeDims / 2; ++i) v = j == i ? rf.inv[i] : v;
  return v;
}
// Launch timing hooks (no-ops unless lcs_timing_enable(1)).
void timing_before(const char* name, hipStream_t s);
void timing_after(const char* name, hipStream_t s);
}  // namespace lcs

#define LCS_LAUNCH(name, kern, grid, block, shmem, stream, ...)                 \
  do {                                                                          \
    lcs::timing_before(name, stream);                                           \
    hipLaunchKernelGGL(kern, grid, block, shmem, stream, __VA_ARGS__);          \
    lcs::timing_after(name, stream);                                            \
  } while (0)
