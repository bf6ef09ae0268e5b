// Core multi-query attention over compressed entries plus the sliding window, with a per-head sink
// (page 1, "hybrid attention": CSA step 3, the HCA paragraph, Q/KV normalization, partial RoPE with
// the output rotated by -i, the sliding-window branch, the attention sink; page 4 section 3.1).
//
// For a query at token t and head h:  qhat = RoPE_t(RMSNorm(q_h)),  l_j = scale * qhat . k_j,
// o_h = sum_j e^{l_j} k_j / (e^{z_h} + sum_j e^{l_j})  (K = V),  then o_h[448:] rotated by -t.
// Keys: the selected entries (CSA) or every visible entry (HCA), followed by tokens [t-W+1, t].
//
// All query heads share each 1 KiB K=V row, so per key the work is 64 heads x 512 dims twice
// (QK^T and PV): ~128 flop per byte, above the fp32-vector ridge, hence bf16 MFMA for both.
// Workgroup = 4 waves = all 64 head slots of one query; keys in tiles of 32.
//   - wave w loads dims [128w, 128w+128) of each tile key from HBM (16 B per lane) and stores
//     the slice in LDS, so the tile is read from HBM once;
//   - QK^T: wave w computes the logits of head block w (heads 16w..16w+15) over all 512 dims,
//     K fragments from the four LDS slices, qhat fragments held in registers;
//   - it runs the online softmax of its 16 heads in registers and publishes P (bf16) and the
//     per-head rescale factors through LDS;
//   - PV: wave w accumulates O[all heads, its 128 dims] += P V, V read from its own LDS slice
//     (laid out so the key-major V fragment reads hit distinct banks).
// The loop is software-pipelined with one barrier per tile: while tile t is scored, tile t-1 is
// accumulated, tile t+1 is moved from registers to LDS and tiles t+2, t+3 are in flight from HBM.
// Keys are split across workgroups (split-K); partial (max, sum, O) are merged by merge_kernel,
// which adds the sink once.  With one split the workgroup finishes the output itself.
#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kTile = 32;                 // keys per tile
constexpr int kWaves = 4;                 // waves per workgroup = 16-head blocks = 128-dim slices
constexpr int kHeadSlots = 16 * kWaves;   // heads handled by one workgroup (all of them)
constexpr int kMaxSplitKeys = 2048;       // keys of one split, staged as row indices in LDS
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 GU32x4;   // global address space: global_load, not flat
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 GU32x2;
typedef __bf16 bf16x2_cv __attribute__((ext_vector_type(2)));
constexpr int kVtStride = 136;            // bf16 per LDS row of a 128-dim slice (128 + 8 pad: rows 4 banks apart)
constexpr float kLog2e = 1.4426950408889634f;
typedef short v4i16 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) v4i16 LdsV4i16;   // LDS operand of the transpose read
typedef __attribute__((address_space(3))) const uint16_t LdsU16;

struct AttnK {
  const uint16_t* q; const uint16_t* gamma_q;
  const uint16_t* kv; int64_t kv_ld;
  const uint8_t* kv8; const float* kv_scale;     // fp8 K=V: E4M3FN codes [.., 512] + one scale per row
  const uint8_t* win8; const float* win_scale;
  const int32_t* topk; int k;
  int64_t n_cap; int m;
  const uint16_t* win; int64_t win_ld, ring_cap; int window;
  const float* sink; const int64_t* q_pos; int64_t rope_offset;
  int Tq, H; float scale_log2, eps;
  RopeFreq rf;
  uint16_t* out; uint16_t* part_o; float* part_ml;
  int nsplit, keys_per_split;
};

// LDS row of tile key (block kb, row r16 of the 16x16 MFMA block) in a slice: the key itself.  With
// rows 272 B apart, the 16 rows a K-fragment read touches start 4 banks apart (no conflicts).
__device__ __forceinline__ int vt_row(int kb, int r16) { return kb * 16 + r16; }

// Four E4M3FN codes (dims 4j .. 4j+3 of a chunk) -> two bf16 pairs, exactly (every E4M3FN value is a
// bf16 value): the gfx950 conversion with unit scale, byte 0 to the low half.
__device__ __forceinline__ uint2 e4m3x4_to_bf16(uint32_t c) {
  return make_uint2(__builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, false)),
                    __builtin_bit_cast(uint32_t, __builtin_amdgcn_cvt_scalef32_pk_bf16_fp8(c, 1.0f, true)));
}

// F8: the K=V rows (compressed entries and window ring) are E4M3FN codes with one fp32 scale per row;
// tiles are converted to bf16 (exactly) when staged in LDS, and each key's scale multiplies its
// logit and, for PV, its probability (o = sum_j p_j s_j code_j), so the MFMAs are those of the bf16
// path on the codes.
template <bool LIST, bool F8>
__global__ void __launch_bounds__(256, 1)
attend_kernel(AttnK a) {
  __shared__ uint16_t s_kv[2][kWaves][kTile * kVtStride];  // tile slices [slot][slice]
  __shared__ uint4 s_p[2][kWaves * kWave];                  // P fragments [slot][head block][lane]
  __shared__ uint4 s_gamma[kHeadDim / 8];                  // gamma_q (bf16)
  __shared__ int s_redo;                                    // some head's running max jumped: second pass
  __shared__ float s_fac[kHeadSlots];
  __shared__ float s_cos[32], s_sin[32];
  __shared__ int32_t s_rows[kMaxSplitKeys];                 // per key of this split: cache/ring row, -1 = none
  __shared__ float4 s_sc[kWaves][2][kTile / 4];             // F8: each wave's copy of the tile's key scales

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t r = blockIdx.y;
  const int64_t b = r / a.Tq;
  const int split = blockIdx.x;
  const int head = 16 * w + c16;          // this lane's head in QK^T and the softmax
  const bool head_ok = head < a.H;

  // Key slots of a row: CSA takes the k list slots (entries < 0 are skipped) then the window tokens,
  // at fixed positions, so a split's range needs no scan of the list; HCA takes the n_vis visible
  // entries then the window tokens.
  const int64_t e_begin = (int64_t)split * a.keys_per_split;
  if (threadIdx.x == 0) s_redo = 0;          // read after the first pass's last barrier

  const uint16_t* kv_b = a.kv + b * a.kv_ld * kHeadDim;
  const int64_t t_q = a.q_pos[r];                         // first load: the RoPE table waits for it alone
  // HCA: the first two tiles are loaded speculatively at once, as entries e_begin .. e_begin+63
  // (clamped into the cache); that holds whenever the split starts with 64 visible entries, which
  // is checked once the query position is known (otherwise they are loaded again).
  uint4 kb0[2][4], kb1[2][4];
  float sc0[2] = {1.f, 1.f}, sc1[2] = {1.f, 1.f};           // F8: scales of the buffers' keys kb*16 + c16
  uint32_t vb0 = 0, vb1 = 0;
  if (!LIST && F8) {
    const uint8_t* kv8_b = a.kv8 + b * a.kv_ld * kHeadDim;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      int64_t e0 = e_begin + kb * 16 + c16, e1 = e0 + kTile;
      e0 = e0 < a.kv_ld ? e0 : a.kv_ld - 1;
      e1 = e1 < a.kv_ld ? e1 : a.kv_ld - 1;
      GU32x2* p0 = reinterpret_cast<GU32x2*>(reinterpret_cast<uintptr_t>(kv8_b + e0 * kHeadDim + 128 * w + 8 * g));
      GU32x2* p1 = reinterpret_cast<GU32x2*>(reinterpret_cast<uintptr_t>(kv8_b + e1 * kHeadDim + 128 * w + 8 * g));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x2 x = p0[4 * ks];
        kb0[kb][ks] = make_uint4(x.x, x.y, 0u, 0u);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x2 x = p1[4 * ks];
        kb1[kb][ks] = make_uint4(x.x, x.y, 0u, 0u);
      }
      sc0[kb] = a.kv_scale[b * a.kv_ld + e0];
      sc1[kb] = a.kv_scale[b * a.kv_ld + e1];
    }
  } else if (!LIST) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int64_t e0 = e_begin + kb * 16 + c16, e1 = e0 + kTile;
      GU32x4* p0 = reinterpret_cast<GU32x4*>(reinterpret_cast<uintptr_t>(
          kv_b + (e0 < a.kv_ld ? e0 : a.kv_ld - 1) * kHeadDim + 128 * w + 8 * g));
      GU32x4* p1 = reinterpret_cast<GU32x4*>(reinterpret_cast<uintptr_t>(
          kv_b + (e1 < a.kv_ld ? e1 : a.kv_ld - 1) * kHeadDim + 128 * w + 8 * g));
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 x = p0[4 * ks];
        kb0[kb][ks] = make_uint4(x.x, x.y, x.z, x.w);
      }
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) {
        const u32x4 x = p1[4 * ks];
        kb1[kb][ks] = make_uint4(x.x, x.y, x.z, x.w);
      }
    }
  }

  // ---- one round trip: this split's list slots, q and gamma ----
  constexpr int kPer = kMaxSplitKeys / 256;
  int32_t sel[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {                        // unconditional (clamped) loads
    const int64_t e = e_begin + threadIdx.x + 256 * u;
    const bool in = e < a.k && threadIdx.x + 256 * u < a.keys_per_split;
    sel[u] = LIST ? a.topk[r * a.k + (in ? e : 0)] : 0;
  }
  // qhat B fragments: lane holds head c16 of block w, dims 32kk + 8g .. +8 for kk = 0..15
  uint4 qf[16];
  {
    const uint16_t* qrow = a.q + (r * a.H + (head_ok ? head : a.H - 1)) * kHeadDim + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
  }
  const uint4 gam = *reinterpret_cast<const uint4*>(a.gamma_q + 8 * (threadIdx.x % (kHeadDim / 8)));
  __builtin_amdgcn_sched_barrier(0);

  // rope table for this query position (same angles for every head), while the rest is in flight
  const double pos = (double)(t_q + a.rope_offset);
  if (threadIdx.x < 32) {
    float cs, sn;
    rope_cs(pos, a.rf.inv[threadIdx.x], &cs, &sn);
    s_cos[threadIdx.x] = cs;
    s_sin[threadIdx.x] = sn;
  }

  int64_t nc;                                             // compressed key slots of the row
  if (LIST) {
    nc = a.k;
  } else {
    const int64_t nv = t_q >= 0 ? t_q / a.m : 0;
    nc = nv < a.n_cap ? nv : a.n_cap;
  }
  const int64_t nk = nc + a.window;
  int64_t e_end = e_begin + a.keys_per_split;
  if (e_end > nk) e_end = nk;
  const int ntiles = e_end > e_begin ? (int)((e_end - e_begin + kTile - 1) / kTile) : 0;
  const int nkeys = e_end > e_begin ? (int)(e_end - e_begin) : 0;

  // ---- the split's key rows: list entry or entry number, then window tokens (ring row); -1 where a
  //      key does not exist ----
  {
    const int64_t j0 = t_q - a.window + 1;                // first window token
    // ring row of token j0 + off (0 <= off < window <= ring_cap): one modulo per row
    const int64_t jm0 = a.ring_cap > 0 && j0 > 0 ? j0 % a.ring_cap : j0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = threadIdx.x + 256 * u;
      const int64_t e = e_begin + i;
      const int64_t off = e - nc;              // window slot
      int64_t jr = jm0 + off;                  // j0 < 0: the token itself (< window <= ring_cap)
      if (a.ring_cap > 0 && jr >= a.ring_cap) jr -= a.ring_cap;
      const int32_t wrow = j0 + off < 0 ? -1 : (int32_t)jr;
      // a negative list entry is no key; so is one past the cache (an unfilled slot must not be read)
      const int32_t crow = LIST ? (sel[u] >= 0 && sel[u] < a.kv_ld ? sel[u] : -1) : (int32_t)e;
      s_rows[i] = i >= nkeys ? -1 : (e < nc ? crow : wrow);
    }
  }
  if (threadIdx.x < kHeadDim / 8) s_gamma[threadIdx.x] = gam;   // gamma: 1 KiB, staged once in LDS
  __syncthreads();
  const uint16_t* win_b = a.win ? a.win + b * a.win_ld * kHeadDim : a.kv;
  const int nc_local = nc > e_begin ? (int)(nc - e_begin) : 0;   // split keys that are compressed

  // ---- tile loads: lane (g, c16) fetches dims 128w + 32ks + 8g of keys kb*16 + c16 ----
  // rows of keys kb*16 + c16 (s_rows is -1 past the split's keys; i0 + 32 <= kMaxSplitKeys)
  auto tile_rows = [&](int i0, int32_t (&rr)[2], uint32_t& vmask) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) rr[kb] = s_rows[i0 + kb * 16 + c16];
    const uint32_t b0 = (uint32_t)__ballot(rr[0] >= 0), b1 = (uint32_t)__ballot(rr[1] >= 0);
    vmask = (b0 & 0xFFFFu) | (b1 << 16);   // bit j: key j of the tile exists (lanes 0..15 hold keys c16)
  };
  auto issue_tile = [&](int i0, const int32_t (&rr)[2], uint4 (&kf)[2][4], float (&sf)[2]) {
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const bool comp = (i0 + kb * 16 + c16) < nc_local;
      const int64_t row = rr[kb] > 0 ? rr[kb] : 0;   // always a readable row (row 0 when the key does not exist)
      if (F8) {
        const uint8_t* base = comp ? a.kv8 + b * a.kv_ld * kHeadDim : a.win8 + b * a.win_ld * kHeadDim;
        GU32x2* p = reinterpret_cast<GU32x2*>(reinterpret_cast<uintptr_t>(base + row * kHeadDim + 128 * w + 8 * g));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x2 x = p[4 * ks];
          kf[kb][ks] = make_uint4(x.x, x.y, 0u, 0u);
        }
        sf[kb] = comp ? a.kv_scale[b * a.kv_ld + row] : a.win_scale[b * a.win_ld + row];
      } else {
        const uint16_t* base = comp ? kv_b : win_b;
        // no predicated loads
        GU32x4* p = reinterpret_cast<GU32x4*>(reinterpret_cast<uintptr_t>(base + row * kHeadDim + 128 * w + 8 * g));
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 x = p[4 * ks];
          kf[kb][ks] = make_uint4(x.x, x.y, x.z, x.w);
        }
      }
    }
  };
  auto load_tile = [&](int i0, uint4 (&kf)[2][4], float (&sf)[2], uint32_t& vmask) {
    int32_t rr[2];
    tile_rows(i0, rr, vmask);
    issue_tile(i0, rr, kf, sf);
  };
  // Two register buffers; an empty split reads row 0.  A load past the end re-reads the last
  // tile, whose copy is never scored.
  auto tile0 = [&](int t) { return (t < ntiles ? t : (ntiles > 0 ? ntiles - 1 : 0)) * kTile; };
  if (!LIST && nkeys >= 2 * kTile && nc_local >= 2 * kTile) {
    vb0 = 0xFFFFFFFFu;                     // the speculative loads are these tiles
    vb1 = 0xFFFFFFFFu;
  } else {
    int32_t r0[2], r1[2];
    tile_rows(tile0(0), r0, vb0);
    tile_rows(tile0(1), r1, vb1);
    issue_tile(tile0(0), r0, kb0, sc0);
    issue_tile(tile0(1), r1, kb1, sc1);
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- qhat = RoPE(RMSNorm(q) * gamma) for head c16 of block w (zero for a padding head) ----
  {
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint4 x = qf[kk];
      const float v[8] = {bf2f_lo(x.x), bf2f_hi(x.x), bf2f_lo(x.y), bf2f_hi(x.y),
                          bf2f_lo(x.z), bf2f_hi(x.z), bf2f_lo(x.w), bf2f_hi(x.w)};
#pragma unroll
      for (int j = 0; j < 8; ++j) acc += v[j] * v[j];
    }
    acc = sum_rows4(acc);
    const float rstd = head_ok ? 1.0f / sqrtf(acc * (1.0f / kHeadDim) + a.eps) : 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int d = 32 * kk + 8 * g;
      const uint4 x = qf[kk];
      const uint4 gm = s_gamma[4 * kk + g];   // dims 32kk + 8g .. +8
      float v[8] = {bf2f_lo(x.x), bf2f_hi(x.x), bf2f_lo(x.y), bf2f_hi(x.y),
                    bf2f_lo(x.z), bf2f_hi(x.z), bf2f_lo(x.w), bf2f_hi(x.w)};
      const float gv[8] = {bf2f_lo(gm.x), bf2f_hi(gm.x), bf2f_lo(gm.y), bf2f_hi(gm.y),
                           bf2f_lo(gm.z), bf2f_hi(gm.z), bf2f_lo(gm.w), bf2f_hi(gm.w)};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * rstd * gv[j];
      if (d >= kRopeStart) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int jr = (d + 2 * p - kRopeStart) >> 1;
          const float cs = s_cos[jr], sn = s_sin[jr];
          const float a0 = v[2 * p], a1 = v[2 * p + 1];
          v[2 * p] = a0 * cs - a1 * sn;
          v[2 * p + 1] = a0 * sn + a1 * cs;
        }
      }
      qf[kk] = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
    }
  }

  floatx4 o[kWaves][8];                    // O^T tiles: lane holds head 16hb + c16, dims 128w + 16db + 4g .. +4
  // Softmax state of this lane's head, log2 domain.  m_ref is the reference of the exponentials:
  // the first tile's max (first pass) or the split's max (second pass); it never moves within a
  // pass, so O is only ever touched by MFMA.  A tile whose max exceeds m_ref by more than kJump
  // (p could pass 2^kJump) makes the first pass void, and the split is run again with m_ref = the
  // split's max, which the first pass has found.
  constexpr float kJump = 16.f;
  float m_ref = -INFINITY, l_run = 0.f, m_max = -INFINITY;
  bool jumped = false;

  // Tile registers -> this wave's LDS slice of `slot` (invalid keys zeroed), then the buffer is
  // refilled with the tile at next_i0, whose rows rn and mask vn were looked up earlier.  Returns
  // the staged tile's key mask.
  auto stage = [&](uint4 (&kf)[2][4], float (&sf)[2], uint32_t& vmask, int slot, int next_i0,
                   const int32_t (&rn)[2], uint32_t vn) -> uint32_t {
    const uint32_t vm = vmask;
    if (F8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const uint2 lo = e4m3x4_to_bf16(kf[kb][ks].x), hi = e4m3x4_to_bf16(kf[kb][ks].y);
          kf[kb][ks] = make_uint4(lo.x, lo.y, hi.x, hi.y);
        }
        if (g == 0) reinterpret_cast<float*>(s_sc[w][slot])[kb * 16 + c16] = sf[kb];
      }
    }
    if (vm != 0xFFFFFFFFu) {               // ragged or missing keys: zero their rows
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool v = (vm >> (kb * 16 + c16)) & 1u;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) kf[kb][ks] = v ? kf[kb][ks] : make_uint4(0, 0, 0, 0);
      }
    }
    uint16_t* sl = s_kv[slot][w];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int vr = vt_row(kb, c16);
#pragma unroll
      for (int ks = 0; ks < 4; ++ks) *reinterpret_cast<uint4*>(&sl[vr * kVtStride + 32 * ks + 8 * g]) = kf[kb][ks];
    }
    issue_tile(next_i0, rn, kf, sf);
    vmask = vn;
    return vm;
  };

  // Logits of head block w for the tile in `slot`, online softmax, P and rescale factors out.
  auto score = [&](int slot, uint32_t vm) {
    floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    // 8 steps of 64 dims (slice h >> 1, ks 2(h & 1) .. +1): the fragments of step h + 1 are read
    // while the MFMAs of step h run (two sets of 4 fragments, 32 registers)
    auto kread = [&](int h, uint4 (&f)[2][2]) {
      const uint16_t* sl = s_kv[slot][h >> 1];
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb)
          f[kb][j] = *reinterpret_cast<const uint4*>(&sl[vt_row(kb, c16) * kVtStride + 32 * (2 * (h & 1) + j) + 8 * g]);
    };
    uint4 fa[2][2], fb[2][2];
    kread(0, fa);
#pragma unroll
    for (int h = 0; h < 8; h += 2) {
      kread(h + 1, fb);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[kb] = mfma_bf16(fa[kb][j], qf[2 * h + j], acc[kb]);
      __builtin_amdgcn_sched_barrier(0);
      if (h + 2 < 8) kread(h + 2, fa);
      __builtin_amdgcn_sched_barrier(0);
#pragma unroll
      for (int j = 0; j < 2; ++j)
#pragma unroll
        for (int kb = 0; kb < 2; ++kb) acc[kb] = mfma_bf16(fb[kb][j], qf[2 * h + 2 + j], acc[kb]);
      __builtin_amdgcn_sched_barrier(0);
    }
    float sc[2][4];
    float ksc[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};   // F8: scales of keys kb*16 + 4g + i
    if (F8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 f = s_sc[w][slot][kb * 4 + g];
        ksc[kb][0] = f.x; ksc[kb][1] = f.y; ksc[kb][2] = f.z; ksc[kb][3] = f.w;
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const bool v = (vm >> (kb * 16 + 4 * g + i)) & 1u;
        sc[kb][i] = v ? acc[kb][i] * (F8 ? ksc[kb][i] * a.scale_log2 : a.scale_log2) : -INFINITY;
        tmax = fmaxf(tmax, sc[kb][i]);
      }
    tmax = max_rows4(tmax);
    m_max = fmaxf(m_max, tmax);
    if (m_ref == -INFINITY) {
      m_ref = tmax;                        // first tile with a key: nothing accumulated yet
    } else if (tmax > m_ref + kJump) {
      jumped = true;                       // this pass is void (the values below stay finite)
    }
    const float mr = fmaxf(m_ref, tmax - kJump);
    uint32_t pk[4] = {0u, 0u, 0u, 0u};
    float psum = 0.f;
    if (mr != -INFINITY) {
      float pe[8];
#pragma unroll
      for (int kb = 0; kb < 2; ++kb)
#pragma unroll
        for (int i = 0; i < 4; ++i) pe[kb * 4 + i] = exp2f(sc[kb][i] - mr);
      if (F8) {
        // PV weights bf16(p_j s_j); the normaliser sums the same rounded weights over s_j, so
        // numerator and denominator see one rounding of p_j, as in the bf16 path
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          const float s0 = ksc[j >> 1][(2 * j) & 3], s1 = ksc[j >> 1][(2 * j + 1) & 3];
          pk[j] = pack_bf2(pe[2 * j] * s0, pe[2 * j + 1] * s1);
          psum += bf2f_lo(pk[j]) * __builtin_amdgcn_rcpf(s0) + bf2f_hi(pk[j]) * __builtin_amdgcn_rcpf(s1);
        }
      } else {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
          pk[j] = pack_bf2(pe[2 * j], pe[2 * j + 1]);
          psum += bf2f_lo(pk[j]) + bf2f_hi(pk[j]);
        }
      }
    }
    psum = sum_rows4(psum);
    l_run += psum;
    s_p[slot][w * kWave + lane] = make_uint4(pk[0], pk[1], pk[2], pk[3]);
  };

  // O[:, this wave's 128 dims] += P V for the tile in `slot`.
  auto accumulate = [&](int slot) {
    uint4 pf[kWaves];
#pragma unroll
    for (int hb = 0; hb < kWaves; ++hb) pf[hb] = s_p[slot][hb * kWave + lane];
    // V fragment (B operand): lane (g, c16) needs k-slots 8g..8g+7 of dim 16db + c16.  Two LDS
    // transpose reads give it: within each 16-lane group, lane j points at 4 consecutive dims
    // (16db + 4(j & 3)) of the key in k-slot 8g + (j >> 2) (then 8g + 4 + (j >> 2)), and lane i
    // receives element i & 3 of the chunks of lanes (i >> 2) + 4q, q = 0..3, i.e. dim 16db + i of
    // k-slots 8g + q.  k-slot 8g + q is key 4g + q, 8g + 4 + q is key 16 + 4g + q (P's order).
    const LdsU16* vbase = (const LdsU16*)(s_kv[slot][w]) + vt_row(0, 4 * g + (c16 >> 2)) * kVtStride +
                          4 * (c16 & 3);
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const v4i16 lo = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4i16*)(vbase + 16 * db));
      const v4i16 hi = __builtin_amdgcn_ds_read_tr16_b64_v4i16((LdsV4i16*)(vbase + 16 * kVtStride + 16 * db));
      const uint2 l2 = __builtin_bit_cast(uint2, lo), h2 = __builtin_bit_cast(uint2, hi);
      const uint4 vf = make_uint4(l2.x, l2.y, h2.x, h2.y);
#pragma unroll
      for (int hb = 0; hb < kWaves; ++hb) o[hb][db] = mfma_bf16(vf, pf[hb], o[hb][db]);
    }
  };

  // Pipeline: iteration t scores tile t (slot t & 1), accumulates tile t-1 (slot (t-1) & 1), stages
  // tile t+1 into slot (t+1) & 1 (free: tile t-1's reads are done in this wave, and in every other
  // wave before the previous barrier) and issues the loads of tile t+3; one barrier.
  for (int pass = 0;; ++pass) {
    if (pass > 0) {                        // second pass: the first two tiles again
      load_tile(tile0(0), kb0, sc0, vb0);
      load_tile(tile0(1), kb1, sc1, vb1);
      m_ref = m_max;
      l_run = 0.f;
    }
#pragma unroll
    for (int hb = 0; hb < kWaves; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) o[hb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    int32_t rn[2];
    uint32_t vn;
    tile_rows(tile0(2), rn, vn);
    uint32_t vm0 = stage(kb0, sc0, vb0, 0, tile0(2), rn, vn);   // tile 0 -> slot 0, buffer 0 <- tile 2
    uint32_t vm1 = 0;
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      tile_rows(tile0(t + 3), rn, vn);              // row lookups first: their latency hides under QK
      score(0, vm0);
      if (t > 0) accumulate(1);
      vm1 = stage(kb1, sc1, vb1, 1, tile0(t + 3), rn, vn);      // tile t+1 -> slot 1, buffer 1 <- tile t+3
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 >= ntiles) break;
      tile_rows(tile0(t + 4), rn, vn);
      score(1, vm1);
      accumulate(0);
      vm0 = stage(kb0, sc0, vb0, 0, tile0(t + 4), rn, vn);      // tile t+2 -> slot 0, buffer 0 <- tile t+4
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ntiles > 0) accumulate((ntiles - 1) & 1);
    if (jumped) s_redo = 1;
    {
      // this pass's output factor per head: one split finishes here (sink, normalisation); with
      // several, the partials stay unnormalised
      float f = 1.f;
      if (a.nsplit == 1) {
        const float z = head_ok ? a.sink[head] * kLog2e : -INFINITY;
        const float M = fmaxf(m_ref, z);
        f = 0.f;
        if (M != -INFINITY) {
          const float L = l_run * exp2f(m_ref - M) + exp2f(z - M);
          f = exp2f(m_ref - M) / L;
        }
      }
      if (g == 0) s_fac[head] = f;
    }
    __syncthreads();                       // s_redo, s_fac; every wave is past its last tile reads
    if (pass > 0 || s_redo == 0) break;
  }

  // Epilogue.  One split finishes the output here (factor s_fac: sink, normalisation); with
  // several, the split stores its partial O and (max, sum).  Either way the last 64 dims are rotated
  // by -(t + offset) here: the rotation is linear, so rotated partials merge to the rotated output.
  // O goes through LDS ([head][dim] bf16, in the tile buffers) so that the global stores are whole
  // 16 B chunks.
  const bool single = a.nsplit == 1;
  constexpr int kOStride = kHeadDim + 8;   // 520 bf16: the 16 heads of one 8-byte write start 4 banks apart
  uint16_t* s_o = &s_kv[0][0][0];          // [64 heads][kOStride] bf16
  static_assert(sizeof(s_kv) >= kHeadSlots * kOStride * 2, "output staging fits the tile buffers");
#pragma unroll
  for (int hb = 0; hb < kWaves; ++hb) {
    const int hh = hb * 16 + c16;
    const float fac = single ? s_fac[hh] : 1.f;   // partials: factor 1
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 128 * w + 16 * db + 4 * g;     // dims d .. d + 3 of head hh
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = single ? o[hb][db][i] * fac : o[hb][db][i];
      if (w == kWaves - 1 && 16 * db >= kRopeStart - 128 * (kWaves - 1)) {
        // dims >= 448 (last wave, db >= 4): rotate the pairs (d, d + 1), (d + 2, d + 3) by -(t + offset)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int jr = ((d - kRopeStart) >> 1) + p;
          const float cs = s_cos[jr], sn = s_sin[jr];
          const float x = v[2 * p], y = v[2 * p + 1];
          v[2 * p] = x * cs + y * sn;
          v[2 * p + 1] = y * cs - x * sn;
        }
      }
      *reinterpret_cast<uint2*>(&s_o[hh * kOStride + d]) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
    }
  }
  __syncthreads();
  const int64_t base = single ? r * a.H : (r * a.nsplit + split) * a.H;
  uint16_t* dst = single ? a.out : a.part_o;
#pragma unroll
  for (int u = 0; u < kHeadSlots * kHeadDim / 8 / 256; ++u) {   // 16 chunks of 8 dims per thread
    const int hl = 4 * u + w;              // one head per wave per step: the check is uniform
    if (hl < a.H) {
      const uint4 x = *reinterpret_cast<const uint4*>(&s_o[hl * kOStride + 8 * lane]);
      *reinterpret_cast<uint4*>(dst + (base + hl) * kHeadDim + 8 * lane) = x;
    }
  }
  if (!single && g == 0 && head_ok)
    *reinterpret_cast<float2*>(a.part_ml + (base + head) * 2) = make_float2(m_ref, l_run);
}

// Merge split-K partials with the sink: one wave per (query, head), 8 dims per lane, no LDS and no
// barrier.  The lanes hold the splits' maxima (split lane + 64 i), the reference M = max(sink, split
// maxima) is a wave reduction, each split's weight 2^(m_s - M) is formed in the lane that holds it
// and broadcast with readlane, and the partial rows are read in rounds of kMergeChunk splits with
// every load of a round issued before the first FMA.
constexpr int kMergeWaves = 4;             // waves per workgroup
constexpr int kMergeChunk = 16;            // partial rows in flight per lane

__global__ void __launch_bounds__(kMergeWaves * kWave)
merge_kernel(const uint16_t* __restrict__ part_o, const float* __restrict__ part_ml, int R, int nsplit, int H,
             const float* __restrict__ sink, uint16_t* __restrict__ out) {
  const int lane = lane_id();
  const int64_t gw = (int64_t)blockIdx.x * kMergeWaves + threadIdx.x / kWave;
  if (gw >= (int64_t)R * H) return;        // wave-uniform
  const int64_t r = gw / H;
  const int h = (int)(gw % H);
  const float z = sink[h] * kLog2e;
  const int64_t row0 = r * nsplit * H + h;  // split sp's row: row0 + sp * H
  auto o_at = [&](int sp) {                // this lane's 8 dims of split sp's partial
    return *reinterpret_cast<const uint4*>(part_o + (row0 + (int64_t)sp * H) * kHeadDim + 8 * lane);
  };
  auto ml_at = [&](int sp) { return *reinterpret_cast<const float2*>(part_ml + (row0 + (int64_t)sp * H) * 2); };

  uint4 v[kMergeChunk];
#pragma unroll
  for (int u = 0; u < kMergeChunk; ++u) v[u] = o_at(u < nsplit ? u : nsplit - 1);   // in flight early

  float mloc = -INFINITY;
  for (int sp = lane; sp < nsplit; sp += kWave) mloc = fmaxf(mloc, ml_at(sp).x);
  const float M = fmaxf(wave_max(mloc), z);

  float acc[8] = {0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f, 0.f};
  float lloc = 0.f;
  for (int c0 = 0; c0 < nsplit; c0 += kWave) {
    // weights of splits c0 .. c0 + 63, one per lane
    const int sp_l = c0 + lane;
    float f_l = 0.f;
    if (sp_l < nsplit) {
      const float2 ml = ml_at(sp_l);
      f_l = M == -INFINITY ? 0.f : exp2f(ml.x - M);
      lloc += f_l * ml.y;
    }
    const int nb = nsplit - c0 < kWave ? nsplit - c0 : kWave;
    for (int c = 0; c < nb; c += kMergeChunk) {
      if (c0 + c > 0) {
#pragma unroll
        for (int u = 0; u < kMergeChunk; ++u) {
          const int sp = c0 + c + u;
          v[u] = o_at(sp < nsplit ? sp : nsplit - 1);
        }
      }
#pragma unroll
      for (int u = 0; u < kMergeChunk; ++u) {
        // split c0 + c + u's weight, from the lane that formed it (the index is wave-uniform)
        const float fw = c + u < nb ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(f_l), (c + u) & 63)) : 0.f;
        const uint32_t wd[4] = {v[u].x, v[u].y, v[u].z, v[u].w};
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          acc[2 * q] += fw * bf2f_lo(wd[q]);
          acc[2 * q + 1] += fw * bf2f_hi(wd[q]);
        }
      }
    }
  }
  float L = wave_sum(lloc);
  if (z != -INFINITY) L += exp2f(z - M);
  const float inv = L > 0.f ? 1.0f / L : 0.f;      // partials are already rotated
  uint4 o;
  o.x = pack_bf2(acc[0] * inv, acc[1] * inv);
  o.y = pack_bf2(acc[2] * inv, acc[3] * inv);
  o.z = pack_bf2(acc[4] * inv, acc[5] * inv);
  o.w = pack_bf2(acc[6] * inv, acc[7] * inv);
  *reinterpret_cast<uint4*>(out + (r * H + h) * kHeadDim + 8 * lane) = o;
}

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Keys per split: about one workgroup per CU (256) with at least 2 tiles (64 keys) each; every split
// adds a 64 KiB partial (bf16 O of 64 heads) that the merge reads back, so splits are kept few.
int keys_per_split(int R, int64_t max_keys) {
  const int64_t tiles = (max_keys + kTile - 1) / kTile;
  if (tiles <= 0) return kTile;
  int64_t want_splits = (256 + R - 1) / R;
  if (want_splits < 1) want_splits = 1;
  int64_t tps = (tiles + want_splits - 1) / want_splits;
  if (tps < 2) tps = 2;
  if (tps > tiles) tps = tiles;
  if (tps > kMaxSplitKeys / kTile) tps = kMaxSplitKeys / kTile;
  return (int)(tps * kTile);
}

}  // namespace

size_t attend_workspace(int B, int Tq, int H, int64_t max_keys) {
  const int R = B * Tq;
  const int kps = keys_per_split(R, max_keys);
  const int64_t nsplit = max_keys > 0 ? (max_keys + kps - 1) / kps : 1;
  if (nsplit <= 1) return 256;
  return al256((size_t)R * nsplit * H * kHeadDim * 2) + al256((size_t)R * nsplit * H * 2 * 4);
}

int launch_attend(const AttendArgs& x, int64_t max_keys, hipStream_t st) {
  const int R = x.B * x.Tq;
  AttnK a;
  a.q = x.q; a.gamma_q = x.gamma_q; a.kv = x.kv; a.kv_ld = x.kv_ld; a.topk = x.topk; a.k = x.k;
  a.n_cap = x.n_cap; a.m = x.m; a.win = x.win; a.win_ld = x.win_ld; a.ring_cap = x.ring_cap;
  a.window = x.window; a.sink = x.sink; a.q_pos = x.q_pos; a.rope_offset = x.rope_offset;
  a.Tq = x.Tq; a.H = x.H; a.scale_log2 = x.scale * kLog2e; a.eps = x.eps; a.rf = rope_freq(x.theta);
  a.out = x.out;
  a.keys_per_split = keys_per_split(R, max_keys);
  a.nsplit = max_keys > 0 ? (int)((max_keys + a.keys_per_split - 1) / a.keys_per_split) : 1;
  if (a.nsplit < 1) a.nsplit = 1;
  a.part_o = static_cast<uint16_t*>(x.ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(x.ws) +
                                       al256((size_t)R * a.nsplit * x.H * kHeadDim * 2));
  const dim3 grid((unsigned)a.nsplit, (unsigned)R);
  a.kv8 = x.kv8; a.kv_scale = x.kv_scale; a.win8 = x.win8; a.win_scale = x.win_scale;
  const bool f8 = x.kv8 != nullptr;
  if (x.topk) {
    if (f8) LCS_LAUNCH("attend_kernel", (attend_kernel<true, true>), grid, dim3(256), 0, st, a);
    else LCS_LAUNCH("attend_kernel", (attend_kernel<true, false>), grid, dim3(256), 0, st, a);
  } else {
    if (f8) LCS_LAUNCH("attend_kernel", (attend_kernel<false, true>), grid, dim3(256), 0, st, a);
    else LCS_LAUNCH("attend_kernel", (attend_kernel<false, false>), grid, dim3(256), 0, st, a);
  }
  if (a.nsplit > 1) {
    const int64_t waves = (int64_t)R * x.H;
    LCS_LAUNCH("attend_merge_kernel", merge_kernel, dim3((unsigned)((waves + kMergeWaves - 1) / kMergeWaves)),
               dim3(kMergeWaves * kWave), 0, st, a.part_o, a.part_ml, R, a.nsplit, x.H, x.sink, x.out);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
