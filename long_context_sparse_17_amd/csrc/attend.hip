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
// Workgroup = 4 waves covering HB 16-head blocks of one query (HB = 4: all 64 heads; HB = 2: 32
// heads, the two halves of a (query, split) in two workgroups placed on the same XCD so the second
// read of each tile comes from its L2, which halves the split partials for the same number of
// workgroups); one workgroup per CU; keys in tiles of 32.
//   - wave w loads dims [128w, 128w+128) of each tile key from HBM (16 B per lane) and stores
//     the slice in LDS, so the workgroup reads the tile once;
//   - QK^T: HB = 4: wave w computes the logits of head block w over both 16-key blocks of the
//     tile; HB = 2: wave w computes head block w & 1 over key block w >> 1 (all 512 dims, K
//     fragments from the four LDS slices, qhat fragments held in registers);
//   - it runs the online softmax of its heads in registers and publishes P (bf16) through LDS;
//   - PV: wave w accumulates O[the workgroup's heads, its 128 dims] += P V, V read from its own
//     LDS slice (laid out so the key-major V fragment reads hit distinct banks).
// The loop is software-pipelined with one barrier per tile: while tile t is scored, tile t-1 is
// accumulated, tile t+1 is moved from registers to LDS and tile t+2 is in flight from HBM.
// Keys are split across workgroups (split-K); partial (max, sum, O) are merged by merge_kernel,
// which adds the sink once.  With one split the workgroup finishes the output itself.
#include <type_traits>

#include "common.h"
#include "decode_append.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kTile = 32;                 // keys per tile
constexpr int kWaves = 4;                 // waves per workgroup = 128-dim slices
constexpr int kMaxSplitKeys = 2048;       // keys of one split, staged as row indices in LDS
constexpr int kMaxBlockEntries = 2048;    // row blocks (QB > 1): cache entries a bitmap covers
typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(1))) const u32x4 GU32x4;   // global address space: global_load, not flat
typedef unsigned int u32x2 __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(1))) const u32x2 GU32x2;
typedef __bf16 bf16x2_cv __attribute__((ext_vector_type(2)));
constexpr int kVtStride = 136;            // bf16 per LDS row of a 128-dim slice (128 + 8 pad: rows 4 banks apart)
constexpr float kLog2e = 1.4426950408889634f;
constexpr bf16x2_cv kOnes2 = {(__bf16)1.0f, (__bf16)1.0f};
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
  int halves;                          // HB = 2: workgroups per (query, split), 1 (H <= 32) or 2
  int R;                               // query rows
  // HCA with a token append in the same launch (app_rows > 0 extra grid rows of append workgroups):
  // a query whose token the append stores forms that window row itself (see the prologue)
  int app_rows;
  DecodeAppendArgs ap;
  RopeFreq rf_ap;
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
// PAD: some head blocks of a workgroup may hold padding heads only (H < 16 HB per workgroup); they are
// not scored (their P stays zero) and not stored.  Without PAD every head block holds a real head.
// QB > 1 (selected-entry lists of many query rows with H = 64 / QB heads): a workgroup takes QB
// consecutive rows of one sequence, head slot s holding head s % H of row s / H, so all 64 slots
// hold real heads.  Its keys are the union of the rows' list entries (one bitmap per row over the
// cache, at most kMaxBlockEntries entries), ascending, then the union of the rows' windows; each
// slot keeps only the logits of its own row's keys (a per-row mask of every tile).  One split.
template <bool LIST, bool F8, int HB, bool PAD, int QB = 1>
__global__ void __launch_bounds__(256, 1)
attend_kernel(AttnK a) {
  static_assert(QB == 1 || (LIST && HB == 4 && !PAD), "row blocks: selected-entry lists, 64 head slots");
  constexpr int kHeadSlots = 16 * HB;                       // heads of one workgroup
  __shared__ uint16_t s_kv[2][kWaves][kTile * kVtStride];  // tile slices [slot][slice]
  __shared__ uint2 s_p[2][HB * kWave][2];                   // P fragments [slot][head block][lane][key block]
  __shared__ float4 s_gamma[kHeadDim / 4];                 // gamma_q (fp32)
  __shared__ int s_redo;                                    // some head's running max jumped: second pass
  __shared__ float s_fac[kHeadSlots];
  __shared__ float s_cos[QB][32], s_sin[QB][32];           // RoPE table of each row's position
  __shared__ int32_t s_rows[kMaxSplitKeys];                 // per key of this split: cache/ring row, -1 = none
  __shared__ float4 s_sc[F8 ? kWaves : 1][2][kTile / 4];    // F8: each wave's copy of the tile's key scales
  __shared__ float2 s_ml[2][kHeadSlots];                    // HB = 2: (sum, max) of each key-block wave's head

  __shared__ __align__(16) uint16_t s_self[kHeadDim];     // the query's own window row (bf16, or kv8 codes)
  __shared__ float s_self_sc;
  __shared__ uint32_t s_bits[QB][QB > 1 ? kMaxBlockEntries / 32 : 1];   // QB > 1: each row's entries
  __shared__ int s_nu;                                      // QB > 1: entries in the union

  if (!LIST && a.app_rows > 0 && (int)blockIdx.y >= a.R) {
    // an append workgroup: sequence (y - R) * nsplit + x on its first 128 threads
    __shared__ float s_red2[2];
    const int ab = ((int)blockIdx.y - a.R) * (int)gridDim.x + (int)blockIdx.x;
    if (ab >= a.ap.B || threadIdx.x >= dapp::kThreads) return;     // whole waves
    dapp::decode_append_seq(a.ap, a.rf_ap, ab, s_red2);
    return;
  }

  const int lane = lane_id();
  const int w = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  // Grid: (split, row) in (x, y); with two head halves a flat x = 16 j + 8 h + i takes (row, split)
  // number 8 j + i = row * nsplit + split and head half h, so the two halves of a split are 8
  // workgroups apart in dispatch order (the same XCD); numbers past the last are padding (< 16)
  int64_t r = blockIdx.y;
  int split = blockIdx.x, hh = 0;
  if (HB == 2 && a.halves == 2) {
    const int64_t u = 8 * (int64_t)(blockIdx.x >> 4) + (blockIdx.x & 7);
    if (u >= (int64_t)a.R * a.nsplit) return;      // uniform
    r = u / a.nsplit;
    split = (int)(u % a.nsplit);
    hh = (int)(blockIdx.x >> 3) & 1;
  }
  int nrows = 1;                          // QB > 1: rows of the block (fewer in a sequence's last block)
  if (QB > 1) {
    const int nblk = (a.Tq + QB - 1) / QB;
    const int q0 = (int)(blockIdx.y % nblk) * QB;
    r = (int64_t)(blockIdx.y / nblk) * a.Tq + q0;
    nrows = a.Tq - q0 < QB ? a.Tq - q0 : QB;
  }
  const int64_t b = r / a.Tq;
  const int hq = HB == 4 ? w : (w & 1);   // head block this wave scores
  const int kbq = HB == 4 ? 0 : (w >> 1); // HB = 2: the key block of each tile it scores
  const int head0 = 32 * hh;              // first head of the workgroup
  const int hl = 16 * hq + c16;           // this lane's head slot in QK^T and the softmax
  constexpr int kH = 64 / QB;             // QB > 1: the heads of every row
  const int qi = QB > 1 ? hl / kH : 0;    // QB > 1: this lane's row in the block
  const int head = QB > 1 ? hl % kH : head0 + hl;
  const bool head_ok = QB > 1 ? qi < nrows : head < a.H;
  // head blocks of the workgroup that hold a real head (fewer than HB when H < 16 HB): the others are
  // neither scored nor accumulated
  // (QB > 1: every block is scored and accumulated; the slots of rows past a sequence's last row have
  // no key, and are not stored)
  const int nvb = !PAD || a.H - head0 >= 16 * HB ? HB : (a.H - head0 + 15) / 16;

  // Key slots of a row: CSA takes the k list slots (entries < 0 are skipped) then the window tokens,
  // at fixed positions, so a split's range needs no scan of the list; HCA takes the n_vis visible
  // entries then the window tokens.
  const int64_t e_begin = (int64_t)split * a.keys_per_split;
  if (threadIdx.x == 0) s_redo = 0;          // read after the first pass's last barrier
  if (PAD && hq >= nvb) {                     // a padding block's P: zero in both slots, never written again
#pragma unroll
    for (int sl = 0; sl < 2; ++sl) {
      s_p[sl][hq * kWave + lane][0] = make_uint2(0u, 0u);
      s_p[sl][hq * kWave + lane][1] = make_uint2(0u, 0u);
    }
  }

  const uint16_t* kv_b = a.kv + b * a.kv_ld * kHeadDim;
  int64_t t_q = a.q_pos[r];                               // uniform: a scalar load (QB > 1: the last)
  int64_t t_lo = t_q;                                     // QB > 1: the block's first position
  int64_t t_r[QB > 4 ? 2 : 1] = {0};                      // QB > 1: positions of rows g (and g + 4)
  if (QB > 1) {
#pragma unroll
    for (int i = 1; i < QB; ++i) {
      if (i < nrows) {
        const int64_t t = a.q_pos[r + i];
        t_q = t > t_q ? t : t_q;
        t_lo = t < t_lo ? t : t_lo;
      }
    }
#pragma unroll
    for (int h = 0; h < (QB > 4 ? 2 : 1); ++h) {
      const int qr = g + 4 * h < nrows ? g + 4 * h : nrows - 1;
      t_r[h] = a.q_pos[r + qr];
    }
  }
  // with an append in this launch: wave 0 loads the query's raw token first, in case this split
  // holds the query's own window row (known once t is; see below), ahead of every other load
  dapp::RingRowIn self_in;
  if (!LIST && a.app_rows > 0 && w == 0) dapp::ring_row_load(a.ap, (int)(r / a.Tq), self_in);
  // this thread's RoPE frequency (threads < 32).  A selected-entry list: picked from the table with
  // constant indices (scalar loads of the kernel arguments), so the RoPE table and the row list ahead of
  // the first tile loads do not wait behind the q loads, as an indexed vector load would (vector loads
  // complete in order).  Dense ranges issue their first tiles before anything else; there the indexed
  // load, placed at its use, measured faster (the scalar table loads delay the tile loads' issue).
  const double rinv = LIST ? rope_inv(a.rf, (int)(threadIdx.x & 31)) : a.rf.inv[threadIdx.x & 31];
  // HCA: the first NB tiles are loaded speculatively at once, as entries e_begin .. e_begin + 32*NB - 1
  // (clamped into the cache); that holds whenever the split starts with 32*NB visible entries, which
  // is checked once the query position is known (otherwise they are loaded again).
  // Register buffers of tiles in flight beyond the one being staged (the loop is written for 1 or 2).
  // One measured faster than two on every layout and shape: CSA decode attention 16.9 -> 15.9 us
  // (bf16 rows) and 19.1 -> 17.4 us (fp8 rows), HCA 31.3 -> 30.8 us, HCA at 64K context 34.5 -> 32.5
  // us, the 1M chunked prefill 1.093 -> 1.082 ms, the 2K prefill's row blocks 0.110 -> 0.107 ms.
  constexpr int NB = 1;
  uint4 kb0[2][4], kb1[2][4];
  float sc0[2] = {1.f, 1.f}, sc1[2] = {1.f, 1.f};           // F8: scales of the buffers' keys kb*16 + c16
  uint32_t vb0 = 0, vb1 = 0;
  uint32_t lb0 = 0, lb1 = 0;                                 // QB > 1: the buffers' per-row key masks
  int ib0 = 0, ib1 = kTile;                                  // first key (split index) of each buffer's tile
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
      if (NB == 2) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x2 x = p1[4 * ks];
          kb1[kb][ks] = make_uint4(x.x, x.y, 0u, 0u);
        }
      }
      sc0[kb] = a.kv_scale[b * a.kv_ld + e0];
      if (NB == 2) sc1[kb] = a.kv_scale[b * a.kv_ld + e1];
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
      if (NB == 2) {
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const u32x4 x = p1[4 * ks];
          kb1[kb][ks] = make_uint4(x.x, x.y, x.z, x.w);
        }
      }
    }
  }

  // ---- one round trip: this split's list slots, q and gamma ----
  constexpr int kPer = kMaxSplitKeys / 256;
  int32_t sel[kPer];
#pragma unroll
  for (int u = 0; u < kPer; ++u) {                        // unconditional (clamped) loads
    if (256 * u >= a.keys_per_split) break;                // uniform: past the split's key slots
    const int64_t e = e_begin + threadIdx.x + 256 * u;
    const bool in = e < a.k && threadIdx.x + 256 * u < a.keys_per_split;
    sel[u] = LIST && QB == 1 ? a.topk[r * a.k + (in ? e : 0)] : 0;
  }
  // gamma before q: loads complete in order, and the barrier below (which the first tile loads of a
  // selected-entry list wait for) needs gamma, the list and the position, not q
  const uint4 gam = *reinterpret_cast<const uint4*>(a.gamma_q + 8 * (threadIdx.x % (kHeadDim / 8)));
  // qhat B fragments: lane holds head c16 of block w, dims 32kk + 8g .. +8 for kk = 0..15
  uint4 qf[16];
  {
    const int64_t qrw = QB > 1 ? (r + (head_ok ? qi : 0)) * a.H + head : r * a.H + (head_ok ? head : a.H - 1);
    const uint16_t* qrow = a.q + qrw * kHeadDim + 8 * g;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) qf[kk] = *reinterpret_cast<const uint4*>(qrow + 32 * kk);
  }
  __builtin_amdgcn_sched_barrier(0);

  // rope table for this query position (same angles for every head), while the rest is in flight
  // (QB > 1: one table per row, threads 32 qr .. 32 qr + 31 for row qr)
  if (threadIdx.x < 32 * QB) {
    const int qr = QB > 1 ? (int)(threadIdx.x >> 5) : 0;
    const int64_t tq = QB > 1 ? a.q_pos[r + (qr < nrows ? qr : nrows - 1)] : t_q;
    const double pos = (double)(tq + a.rope_offset);
    float cs, sn;
    rope_cs(pos, rinv, &cs, &sn);
    s_cos[qr][threadIdx.x & 31] = cs;
    s_sin[qr][threadIdx.x & 31] = sn;
  }

  // QB > 1: one bitmap per row of its list entries (entries < 0 or past the cache are no key), their
  // union compacted into s_rows in ascending order by wave 0 (lane l: entries 32 l .. 32 l + 31)
  if (QB > 1) {
    constexpr int kWords = kMaxBlockEntries / 32;
    for (int i = threadIdx.x; i < QB * kWords; i += 256) s_bits[i / kWords][i % kWords] = 0u;
    __syncthreads();
    const int n_list = nrows * a.k;
    for (int i0 = 0; i0 < n_list; i0 += 4 * 256) {
      int32_t ev[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {                       // unconditional (clamped) loads
        const int i = i0 + 256 * u + (int)threadIdx.x;
        ev[u] = a.topk[r * a.k + (i < n_list ? i : 0)];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int i = i0 + 256 * u + (int)threadIdx.x;
        const int32_t e = ev[u];
        if (i < n_list && e >= 0 && e < a.kv_ld) atomicOr(&s_bits[i / a.k][e >> 5], 1u << (e & 31));
      }
    }
    __syncthreads();
    if (w == 0) {
      uint32_t un = 0u;
#pragma unroll
      for (int q = 0; q < QB; ++q) un |= s_bits[q][lane];
      const int cnt = __popc(un);
      int incl = cnt;                                     // inclusive prefix over the lanes
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const int v = __shfl_up(incl, o, kWave);
        if (lane >= o) incl += v;
      }
      int at = incl - cnt;
      while (un != 0u) {
        s_rows[at++] = 32 * lane + __ffs(un) - 1;
        un &= un - 1u;
      }
      if (lane == kWave - 1) s_nu = incl;
    }
    __syncthreads();
  }

  int64_t nc;                                             // compressed key slots of the row
  if (QB > 1) {
    nc = s_nu;
  } else if (LIST) {
    nc = a.k;
  } else {
    const int64_t nv = t_q >= 0 ? t_q / a.m : 0;
    nc = nv < a.n_cap ? nv : a.n_cap;
  }
  // QB > 1: the rows' windows as one range of tokens j_lo .. t_q (a token no row uses is no key)
  const int64_t j_lo = QB > 1 ? (t_lo - a.window + 1 > 0 ? t_lo - a.window + 1 : 0) : 0;
  const int64_t nwin = QB > 1 ? (a.window > 0 && t_q >= j_lo ? t_q - j_lo + 1 : 0) : a.window;
  const int64_t nk = nc + nwin;
  int64_t e_end = e_begin + a.keys_per_split;
  if (e_end > nk) e_end = nk;
  const int ntiles = e_end > e_begin ? (int)((e_end - e_begin + kTile - 1) / kTile) : 0;
  const int nkeys = e_end > e_begin ? (int)(e_end - e_begin) : 0;
  // The query's own token, when this launch's append stores it (HCA with an append, pos[b] = t): its
  // window row (the last key, slot nk - 1) is being written to the ring by the append workgroups, so
  // the split that holds it forms the row here, the way the append does, and the staging puts it in
  // place of whatever the ring row read returns.  sk: its index in this split, or -1.
  int sk = -1;
  if (!LIST && a.app_rows > 0 && a.window > 0 && t_q >= 0 && a.ap.pos[b] == t_q) {
    const int64_t s0 = nk - 1 - e_begin;
    if (s0 >= 0 && s0 < nkeys) sk = (int)s0;
  }
  if (sk >= 0 && w == 0) dapp::ring_row_compute(a.ap, a.rf_ap, t_q, self_in, s_self, &s_self_sc);   // before the barrier below

  // ---- the split's key rows: list entry or entry number, then window tokens (ring row); -1 where a
  //      key does not exist (QB > 1: s_rows holds the union's entries; window rows are formed per tile) ----
  if (QB == 1) {
    const int64_t j0 = t_q - a.window + 1;                // first window token
    // ring row of token j0 + off (0 <= off < window <= ring_cap): one modulo per row
    const int64_t jm0 = a.ring_cap > 0 && j0 > 0 ? j0 % a.ring_cap : j0;
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      if (256 * u >= a.keys_per_split) break;              // uniform: tiles read no slot past the split's
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
  if (threadIdx.x < kHeadDim / 8) {          // gamma: staged once in LDS, as fp32
    s_gamma[2 * threadIdx.x] = make_float4(bf2f_lo(gam.x), bf2f_hi(gam.x), bf2f_lo(gam.y), bf2f_hi(gam.y));
    s_gamma[2 * threadIdx.x + 1] = make_float4(bf2f_lo(gam.z), bf2f_hi(gam.z), bf2f_lo(gam.w), bf2f_hi(gam.w));
  }
  __syncthreads();
  const uint16_t* win_b = a.win ? a.win + b * a.win_ld * kHeadDim : a.kv;
  const int nc_local = nc > e_begin ? (int)(nc - e_begin) : 0;   // split keys that are compressed

  // ---- tile loads: lane (g, c16) fetches dims 128w + 32ks + 8g of keys kb*16 + c16 ----
  // QB > 1: ring row of window token j_lo + off (off < nwin); one wrap when nwin <= ring_cap
  const int64_t jm_lo = QB > 1 && a.ring_cap > 0 ? j_lo % a.ring_cap : j_lo;
  const bool wrap_once = a.ring_cap <= 0 || nwin <= a.ring_cap;
  // rows of keys kb*16 + c16 (s_rows is -1 past the split's keys; i0 + 32 <= kMaxSplitKeys).  lmask
  // (QB > 1): bit j is set where key j of the tile is a key of this lane's row; vmask then marks the
  // keys of any row of the block (the others are not keys)
  auto tile_rows = [&](int i0, int32_t (&rr)[2], uint32_t& vmask, uint32_t& lmask) {
    if (QB == 1) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) rr[kb] = s_rows[i0 + kb * 16 + c16];
      const uint32_t b0 = (uint32_t)__ballot(rr[0] >= 0), b1 = (uint32_t)__ballot(rr[1] >= 0);
      vmask = (b0 & 0xFFFFu) | (b1 << 16);   // bit j: key j of the tile exists (lanes 0..15 hold keys c16)
      lmask = vmask;
      return;
    }
    // QB > 1: lane (g, c16) decides key kb*16 + c16 for rows g and g + 4
    constexpr int NH = QB > 4 ? 2 : 1;
    uint64_t bal[2][NH];
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      const int i = i0 + kb * 16 + c16;
      int32_t row = -1;
      int64_t j = -1;                                     // window token, or -1 for an entry
      if (i < nc_local) {
        row = s_rows[i];
      } else if (i < nkeys) {
        const int64_t off = (int64_t)(i - nc_local);
        j = j_lo + off;
        int64_t jr = jm_lo + off;
        if (a.ring_cap > 0) {
          if (wrap_once) jr = jr >= a.ring_cap ? jr - a.ring_cap : jr;
          else jr %= a.ring_cap;
        }
        row = (int32_t)jr;
      }
      rr[kb] = row;
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const int qr = g + 4 * h;
        bool in = false;
        if (qr < nrows && row >= 0) {
          if (j < 0) in = (s_bits[qr][row >> 5] >> (row & 31)) & 1u;
          else in = j > t_r[h] - a.window && j <= t_r[h];
        }
        bal[kb][h] = __ballot(in);
      }
    }
    // row q's bits of key block kb: bits 16 (q & 3) .. +15 of bal[kb][q >> 2]
    uint32_t any[2] = {0u, 0u};
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int h = 0; h < NH; ++h) {
        const uint64_t x = bal[kb][h];
        any[kb] |= (uint32_t)(x | (x >> 16) | (x >> 32) | (x >> 48)) & 0xFFFFu;
      }
    vmask = any[0] | (any[1] << 16);
    const int hsel = qi >> 2, csel = 16 * (qi & 3);
    const uint64_t x0 = NH == 2 && hsel ? bal[0][NH - 1] : bal[0][0];
    const uint64_t x1 = NH == 2 && hsel ? bal[1][NH - 1] : bal[1][0];
    lmask = ((uint32_t)(x0 >> csel) & 0xFFFFu) | (((uint32_t)(x1 >> csel) & 0xFFFFu) << 16);
    // a key of no row is not loaded
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) rr[kb] = (vmask >> (kb * 16 + c16)) & 1u ? rr[kb] : -1;
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
  auto load_tile = [&](int i0, uint4 (&kf)[2][4], float (&sf)[2], uint32_t& vmask, uint32_t& lmask) {
    int32_t rr[2];
    tile_rows(i0, rr, vmask, lmask);
    issue_tile(i0, rr, kf, sf);
  };
  // The register buffers; an empty split reads row 0.  A load past the end re-reads the last
  // tile, whose copy is never scored.
  auto tile0 = [&](int t) { return (t < ntiles ? t : (ntiles > 0 ? ntiles - 1 : 0)) * kTile; };
  if (!LIST && nkeys >= NB * kTile && nc_local >= NB * kTile) {
    vb0 = 0xFFFFFFFFu;                     // the speculative loads are these tiles
    vb1 = 0xFFFFFFFFu;
  } else {
    int32_t r0[2], r1[2];
    ib0 = tile0(0);
    ib1 = tile0(1);
    tile_rows(tile0(0), r0, vb0, lb0);
    issue_tile(tile0(0), r0, kb0, sc0);
    if (NB == 2) {
      tile_rows(tile0(1), r1, vb1, lb1);
      issue_tile(tile0(1), r1, kb1, sc1);
    }
  }
  __builtin_amdgcn_sched_barrier(0);

  // ---- qhat = RoPE(RMSNorm(q) * gamma) for head c16 of block w (zero for a padding head).  The
  //      fragments hold RoPE(q * gamma); the head's 1 / rms, a scalar, multiplies its logits instead
  //      (the rotation is linear), which saves a multiply per element here and costs none there ----
  float lsc;                               // this lane's head: logit scale (log2 domain) / rms
  {
    float acc = 0.f;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const uint4 x = qf[kk];
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_cv, x.x), __builtin_bit_cast(bf16x2_cv, x.x), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_cv, x.y), __builtin_bit_cast(bf16x2_cv, x.y), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_cv, x.z), __builtin_bit_cast(bf16x2_cv, x.z), acc, false);
      acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_cv, x.w), __builtin_bit_cast(bf16x2_cv, x.w), acc, false);
    }
    acc = sum_rows4(acc);
    const float rstd = head_ok ? 1.0f / sqrtf(acc * (1.0f / kHeadDim) + a.eps) : 0.f;
    lsc = a.scale_log2 * rstd;
#pragma unroll
    for (int kk = 0; kk < 16; ++kk) {
      const int d = 32 * kk + 8 * g;
      const uint4 x = qf[kk];
      const float4 g0 = s_gamma[8 * kk + 2 * g], g1 = s_gamma[8 * kk + 2 * g + 1];   // dims 32kk + 8g .. +8
      float v[8] = {bf2f_lo(x.x), bf2f_hi(x.x), bf2f_lo(x.y), bf2f_hi(x.y),
                    bf2f_lo(x.z), bf2f_hi(x.z), bf2f_lo(x.w), bf2f_hi(x.w)};
      const float gv[8] = {g0.x, g0.y, g0.z, g0.w, g1.x, g1.y, g1.z, g1.w};
#pragma unroll
      for (int j = 0; j < 8; ++j) v[j] = v[j] * gv[j];
      if (d >= kRopeStart) {
#pragma unroll
        for (int p = 0; p < 4; ++p) {
          const int jr = (d + 2 * p - kRopeStart) >> 1;
          const float cs = s_cos[qi][jr], sn = s_sin[qi][jr];
          const float a0 = v[2 * p], a1 = v[2 * p + 1];
          v[2 * p] = a0 * cs - a1 * sn;
          v[2 * p + 1] = a0 * sn + a1 * cs;
        }
      }
      qf[kk] = make_uint4(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]), pack_bf2(v[4], v[5]), pack_bf2(v[6], v[7]));
    }
  }

  floatx4 o[HB][8];                        // O^T tiles: lane holds head slot 16hb + c16, dims 128w + 16db + 4g .. +4
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
  auto stage = [&](uint4 (&kf)[2][4], float (&sf)[2], uint32_t& vmask, uint32_t& lmask, int& bi0, int slot,
                   int next_i0, const int32_t (&rn)[2], uint32_t vn, uint32_t ln, uint32_t& lm) -> uint32_t {
    const uint32_t vm = vmask;
    lm = lmask;
    if (sk >= bi0 && sk < bi0 + kTile) {   // uniform: this tile holds the query's own window row
      const int j = sk - bi0;
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        if (kb * 16 + c16 != j) continue;
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
          const int d = 128 * w + 32 * ks + 8 * g;
          if (F8) {
            const uint2 cw = *reinterpret_cast<const uint2*>(reinterpret_cast<const uint8_t*>(s_self) + d);
            kf[kb][ks] = make_uint4(cw.x, cw.y, 0u, 0u);
          } else {
            kf[kb][ks] = *reinterpret_cast<const uint4*>(&s_self[d]);
          }
        }
        if (F8) sf[kb] = s_self_sc;
      }
    }
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
    bi0 = next_i0;
    vmask = vn;
    lmask = ln;
    return vm;
  };

  // Logits of this wave's head block for the tile in `slot`, online softmax, P out.  HB = 4: both
  // key blocks of the tile.  HB = 2: the wave's own key block, except on the first tile with a key
  // of a pass, where both are scored so that the two waves of a head block take the same reference
  // (the same instructions on the same operands: the same bits).
  auto qk = [&](int slot, int kb, floatx4& acc) {
    // 8 steps of 64 dims (slice h >> 1, ks 2(h & 1) .. +1); two accumulation chains (even and odd
    // 32-dim steps) so that consecutive MFMAs are independent; the fragments of step h + 1 are read
    // while the MFMAs of step h run
    floatx4 ae = {0.f, 0.f, 0.f, 0.f}, ao = {0.f, 0.f, 0.f, 0.f};
    auto kread = [&](int h, uint4 (&f)[2]) {
      const uint16_t* sl = s_kv[slot][h >> 1];
#pragma unroll
      for (int j = 0; j < 2; ++j)
        f[j] = *reinterpret_cast<const uint4*>(&sl[vt_row(kb, c16) * kVtStride + 32 * (2 * (h & 1) + j) + 8 * g]);
    };
    uint4 fa[2], fb[2];
    kread(0, fa);
#pragma unroll
    for (int h = 0; h < 8; h += 2) {
      kread(h + 1, fb);
      ae = mfma_bf16(fa[0], qf[2 * h], ae);
      ao = mfma_bf16(fa[1], qf[2 * h + 1], ao);
      if (h + 2 < 8) kread(h + 2, fa);
      ae = mfma_bf16(fb[0], qf[2 * h + 2], ae);
      ao = mfma_bf16(fb[1], qf[2 * h + 3], ao);
    }
    acc = ae + ao;
  };
  auto score = [&](int slot, uint32_t vm, uint32_t lm) {
    if (PAD && hq >= nvb) return;          // wave-uniform: a head block of padding heads only
    floatx4 acc[2] = {floatx4{0.f, 0.f, 0.f, 0.f}, floatx4{0.f, 0.f, 0.f, 0.f}};
    const bool both = HB == 4 || m_ref == -INFINITY;       // uniform: -inf only before a tile with a key
    if (both) {
      qk(slot, 0, acc[0]);
      qk(slot, 1, acc[1]);
    } else {
      qk(slot, kbq, acc[kbq]);
    }
    float sc[2][4];
    float ksc[2][4] = {{1.f, 1.f, 1.f, 1.f}, {1.f, 1.f, 1.f, 1.f}};   // F8: scales of keys kb*16 + 4g + i
    if (F8) {
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const float4 f = s_sc[F8 ? w : 0][slot][kb * 4 + g];
        ksc[kb][0] = f.x; ksc[kb][1] = f.y; ksc[kb][2] = f.z; ksc[kb][3] = f.w;
      }
    }
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) sc[kb][i] = acc[kb][i] * (F8 ? ksc[kb][i] * lsc : lsc);
    if (QB > 1 || vm != 0xFFFFFFFFu || HB == 2) {   // uniform: missing keys, or key blocks not scored here
      const uint32_t mk = QB > 1 ? lm : vm;            // QB > 1: the keys of this lane's row
#pragma unroll
      for (int kb = 0; kb < 2; ++kb) {
        const bool mine = HB == 4 || kb == kbq;
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          const bool v = (both || mine) && ((mk >> (kb * 16 + 4 * g + i)) & 1u);
          sc[kb][i] = v ? sc[kb][i] : -INFINITY;
        }
      }
    }
    float tmax = -INFINITY;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb)
#pragma unroll
      for (int i = 0; i < 4; ++i) tmax = fmaxf(tmax, sc[kb][i]);
    tmax = max_rows4(tmax);
    m_max = fmaxf(m_max, tmax);
    if (m_ref == -INFINITY) {
      m_ref = tmax;                        // first tile with a key: nothing accumulated yet
    } else if (tmax > m_ref + kJump) {
      jumped = true;                       // this pass is void (the values below stay finite)
    }
    const float mr = fmaxf(m_ref, tmax - kJump);
    float psum = 0.f;
#pragma unroll
    for (int kb = 0; kb < 2; ++kb) {
      if (HB == 2 && kb != kbq) continue;  // the other key block is the partner wave's
      uint32_t pk[2] = {0u, 0u};
      if (mr != -INFINITY) {
        float pe[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) pe[i] = __builtin_amdgcn_exp2f(sc[kb][i] - mr);   // arguments <= kJump
        if (F8) {
          // PV weights bf16(p_j s_j); the normaliser sums the same rounded weights over s_j, so
          // numerator and denominator see one rounding of p_j, as in the bf16 path
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            const float s0 = ksc[kb][2 * j], s1 = ksc[kb][2 * j + 1];
            pk[j] = pack_bf2(pe[2 * j] * s0, pe[2 * j + 1] * s1);
            psum += bf2f_lo(pk[j]) * __builtin_amdgcn_rcpf(s0) + bf2f_hi(pk[j]) * __builtin_amdgcn_rcpf(s1);
          }
        } else {
#pragma unroll
          for (int j = 0; j < 2; ++j) {
            pk[j] = pack_bf2(pe[2 * j], pe[2 * j + 1]);
            psum = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2_cv, pk[j]), kOnes2, psum, false);
          }
        }
      }
      s_p[slot][hq * kWave + lane][kb] = make_uint2(pk[0], pk[1]);
    }
    psum = sum_rows4(psum);
    l_run += psum;
  };

  // O[:, this wave's 128 dims] += P V for the tile in `slot`.
  // NV: the head blocks accumulated (a compile-time count, so the full case has no per-block test)
  auto accumulate_nv = [&](int slot, auto nv_c) {
    constexpr int NV = decltype(nv_c)::value;
    uint4 pf[HB];
#pragma unroll
    for (int hb = 0; hb < NV; ++hb) {
      const uint2 lo = s_p[slot][hb * kWave + lane][0], hi = s_p[slot][hb * kWave + lane][1];
      pf[hb] = make_uint4(lo.x, lo.y, hi.x, hi.y);
    }
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
      for (int hb = 0; hb < NV; ++hb) o[hb][db] = mfma_bf16(vf, pf[hb], o[hb][db]);
    }
  };
  // Every head block is accumulated (the padding blocks' P is zero): choosing the block count per call
  // would make the compiler move the accumulators between register assignments in the loop.
  auto accumulate = [&](int slot) { accumulate_nv(slot, std::integral_constant<int, HB>{}); };

  // Pipeline: iteration t scores tile t (slot t & 1), accumulates tile t-1 (slot (t-1) & 1), stages
  // tile t+1 into slot (t+1) & 1 (free: tile t-1's V reads are done in this wave, which reads only
  // its own slice, and every wave's K reads of it before the previous barrier) and issues the loads
  // of tile t+1+NB; one barrier.
  for (int pass = 0;; ++pass) {
    if (pass > 0) {                        // second pass: the first tiles again
      load_tile(tile0(0), kb0, sc0, vb0, lb0);
      ib0 = tile0(0);
      if (NB == 2) { load_tile(tile0(1), kb1, sc1, vb1, lb1); ib1 = tile0(1); }
      m_ref = m_max;                       // the split's max (HB = 2: over both key-block waves)
      l_run = 0.f;
    }
#pragma unroll
    for (int hb = 0; hb < HB; ++hb)
#pragma unroll
      for (int db = 0; db < 8; ++db) o[hb][db] = floatx4{0.f, 0.f, 0.f, 0.f};
    int32_t rn[2];
    uint32_t vn, ln, lm0, lm1 = 0;
    tile_rows(tile0(NB), rn, vn, ln);
    uint32_t vm0 = stage(kb0, sc0, vb0, lb0, ib0, 0, tile0(NB), rn, vn, ln, lm0);  // tile 0 -> slot 0, buffer 0 <- tile NB
    uint32_t vm1 = 0;
    __syncthreads();
    for (int t = 0; t < ntiles; t += 2) {
      tile_rows(tile0(t + 1 + NB), rn, vn, ln);     // row lookups first: their latency hides under QK
      score(0, vm0, lm0);
      if (t > 0) accumulate(1);
      // tile t+1 -> slot 1; its buffer <- tile t+1+NB
      if (NB == 2) vm1 = stage(kb1, sc1, vb1, lb1, ib1, 1, tile0(t + 3), rn, vn, ln, lm1);
      else vm1 = stage(kb0, sc0, vb0, lb0, ib0, 1, tile0(t + 2), rn, vn, ln, lm1);
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
      if (t + 1 >= ntiles) break;
      tile_rows(tile0(t + 2 + NB), rn, vn, ln);
      score(1, vm1, lm1);
      accumulate(0);
      vm0 = stage(kb0, sc0, vb0, lb0, ib0, 0, tile0(t + 2 + NB), rn, vn, ln, lm0);  // tile t+2 -> slot 0, buffer 0 <- tile t+2+NB
      __syncthreads();
      __builtin_amdgcn_sched_barrier(0);
    }
    if (ntiles > 0) accumulate((ntiles - 1) & 1);
    if (jumped) s_redo = 1;
    if (HB == 2 && g == 0) s_ml[kbq][hl] = make_float2(l_run, m_max);
    __syncthreads();                       // s_redo, s_ml; every wave is past its last tile reads
    if (HB == 2) {                         // the partner wave's keys: same reference, its own sum and max
      const float2 o2 = s_ml[kbq ^ 1][hl];
      l_run += o2.x;
      m_max = fmaxf(m_max, o2.y);
    }
    if (pass > 0 || s_redo == 0) break;
  }
  {
    // the output factor per head: one split finishes here (sink, normalisation); with several, the
    // partials stay unnormalised
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
    if (g == 0 && kbq == 0) s_fac[hl] = f;
  }
  __syncthreads();                         // s_fac

  // Epilogue.  One split finishes the output here (factor s_fac: sink, normalisation); with
  // several, the split stores its partial O and (max, sum).  Either way the last 64 dims are rotated
  // by -(t + offset) here: the rotation is linear, so rotated partials merge to the rotated output.
  // O goes through LDS ([head][dim] bf16, in the tile buffers) so that the global stores are whole
  // 16 B chunks.
  const bool single = a.nsplit == 1;
  constexpr int kOStride = kHeadDim + 8;   // 520 bf16: the 16 heads of one 8-byte write start 4 banks apart
  uint16_t* s_o = &s_kv[0][0][0];          // [head slots][kOStride] bf16
  static_assert(sizeof(s_kv) >= kHeadSlots * kOStride * 2, "output staging fits the tile buffers");
#pragma unroll
  for (int hb = 0; hb < HB; ++hb) {
    if (PAD && hb >= nvb) break;           // uniform: padding heads are not stored
    const int hh = hb * 16 + c16;
    const float fac = single ? s_fac[hh] : 1.f;   // partials: factor 1 (exact)
#pragma unroll
    for (int db = 0; db < 8; ++db) {
      const int d = 128 * w + 16 * db + 4 * g;     // dims d .. d + 3 of head hh
      float v[4];
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = o[hb][db][i] * fac;
      if (w == kWaves - 1 && 16 * db >= kRopeStart - 128 * (kWaves - 1)) {
        // dims >= 448 (last wave, db >= 4): rotate the pairs (d, d + 1), (d + 2, d + 3) by -(t + offset)
#pragma unroll
        for (int p = 0; p < 2; ++p) {
          const int jr = ((d - kRopeStart) >> 1) + p;
          const int qo = QB > 1 ? hh / kH : 0;
          const float cs = s_cos[qo][jr], sn = s_sin[qo][jr];
          const float x = v[2 * p], y = v[2 * p + 1];
          v[2 * p] = x * cs + y * sn;
          v[2 * p + 1] = y * cs - x * sn;
        }
      }
      *reinterpret_cast<uint2*>(&s_o[hh * kOStride + d]) = make_uint2(pack_bf2(v[0], v[1]), pack_bf2(v[2], v[3]));
    }
  }
  __syncthreads();
  const int64_t base = (single ? r * a.H : (r * a.nsplit + split) * a.H) + head0;
  uint16_t* dst = single ? a.out : a.part_o;
  // Split partials are read once, by the merge launch, on whichever XCD its workgroup lands: they are
  // stored non-temporally, so they do not hold L2 lines that the next launches' reads would have to
  // evict (measured: the decode step gains about 2 %, most of it in the next indexer launch)
#pragma unroll
  for (int u = 0; u < kHeadSlots * kHeadDim / 8 / 256; ++u) {   // HB * 4 chunks of 8 dims per thread
    const int ho = 4 * u + w;              // one head per wave per step: the check is uniform
    if (QB > 1 ? ho < nrows * kH : head0 + ho < a.H) {
      const u32x4 x = *reinterpret_cast<const u32x4*>(&s_o[ho * kOStride + 8 * lane]);
      u32x4* at = reinterpret_cast<u32x4*>(dst + (base + ho) * kHeadDim + 8 * lane);
      if (single) *at = x;
      else __builtin_nontemporal_store(x, at);
    }
  }
  if (!single && g == 0 && kbq == 0 && head_ok)
    *reinterpret_cast<float2*>(a.part_ml + (base + hl) * 2) = make_float2(m_ref, l_run);
}

// Merge split-K partials with the sink: one wave per (query, head), 8 dims per lane, no LDS and no
// barrier.  The lanes hold the splits' maxima (split lane + 64 i), the reference M = max(sink, split
// maxima) is a wave reduction, each split's weight 2^(m_s - M) is formed in the lane that holds it
// and broadcast with readlane, and the partial rows are read in rounds of kMergeChunk splits with
// every load of a round issued before the first FMA.  kMergeChunk (partial rows in flight per lane)
// is 4, 8 or 16, the smallest that holds the call's splits (up to 16): loads past the last split
// repeat its row, so a round sized to the split count issues none of them (HCA at 64K context, 4
// splits: 32.8 -> 29.9 us per call).
constexpr int kMergeWaves = 4;             // waves per workgroup
template <int kMergeChunk>
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
  auto o_at = [&](int sp) {                // this lane's 8 dims of split sp's partial (read once: non-temporal)
    const u32x4 x = __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(part_o + (row0 + (int64_t)sp * H) * kHeadDim + 8 * lane));
    return make_uint4(x.x, x.y, x.z, x.w);
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

// Keys per split: about one workgroup per CU (256, counting both head halves with HB = 2) with at
// least 2 tiles (64 keys) each.  Every split adds a 64 KiB partial (bf16 O of 64 heads) that the
// merge reads back, so splits are kept few.
template <int HB>
int keys_per_split(int R, int halves, int64_t max_keys) {
  const int64_t tiles = (max_keys + kTile - 1) / kTile;
  if (tiles <= 0) return kTile;
  const int64_t slots = 256;
  int64_t want_splits = (slots + (int64_t)R * halves - 1) / ((int64_t)R * halves);
  if (want_splits < 1) want_splits = 1;
  int64_t tps = (tiles + want_splits - 1) / want_splits;
  if (tps < 2) tps = 2;
  if (tps > tiles) tps = tiles;
  if (tps > kMaxSplitKeys / kTile) tps = kMaxSplitKeys / kTile;
  return (int)(tps * kTile);
}

// The layout a call runs with.  Selected entries (CSA) of few query rows (decode): HB = 2, whose
// halved split partials cut the epilogue and merge that dominate a short key list.  At most 32 heads:
// HB = 2 too (32 head slots hold every head; 64 would be half padding or more).  All visible entries
// (HCA) and many rows (prefill, one split per row) of more heads: HB = 4, whose loop keeps twice the
// unique bytes in flight per CU and reads each tile once.
struct AttendPlan {
  int hb, halves, keys_per_split, nsplit;
};
AttendPlan attend_plan(int R, int H, int64_t max_keys, bool list) {
  AttendPlan p;
  p.hb = (list && R < 128) || H <= 32 ? 2 : 4;   // H <= 32: 32 head slots are enough
  p.halves = p.hb == 2 && H > 32 ? 2 : 1;
  p.keys_per_split = p.hb == 2 ? keys_per_split<2>(R, p.halves, max_keys) : keys_per_split<4>(R, 1, max_keys);
  p.nsplit = max_keys > 0 ? (int)((max_keys + p.keys_per_split - 1) / p.keys_per_split) : 1;
  if (p.nsplit < 1) p.nsplit = 1;
  return p;
}

}  // namespace

size_t attend_workspace(int B, int Tq, int H, int64_t max_keys) {
  // one query serves both entry points: the larger of the two layouts' split partials
  const int R = B * Tq;
  int nsplit = 1;
  for (int list = 0; list < 2; ++list) {
    const AttendPlan p = attend_plan(R, H, max_keys, list != 0);
    nsplit = p.nsplit > nsplit ? p.nsplit : nsplit;
  }
  if (nsplit <= 1) return 256;
  return al256((size_t)R * nsplit * H * kHeadDim * 2) + al256((size_t)R * nsplit * H * 2 * 4);
}

// Every grid the call would launch fits the HIP limits (the flat grid of two head halves: x < 2^31).
bool attend_launchable(int B, int Tq, int H, int64_t max_keys, bool list) {
  const int R = B * Tq;
  const AttendPlan p = attend_plan(R, H, max_keys, list);
  if (p.hb == 2 && p.halves == 2) return 16 * (((int64_t)R * p.nsplit + 7) / 8) < ((int64_t)1 << 31);
  return p.nsplit < ((int64_t)1 << 31);
}

// Rows per workgroup: QB > 1 for selected-entry lists of many rows (prefill) with few heads (H = 64 /
// QB, QB = 2, 4 or 8) over a cache of at most kMaxBlockEntries entries, whose rows' lists overlap
// enough that their union is far shorter than QB lists.  Else 1.
int attend_rows_per_block(int B, int Tq, int H, int64_t kv_ld, bool list, bool append) {
  if (!list || append || (int64_t)B * Tq < 128 || kv_ld > kMaxBlockEntries) return 1;
  if (H != 8 && H != 16 && H != 32) return 1;
  const int qb = 64 / H;
  return Tq >= qb ? qb : 1;
}

template <bool LIST, bool F8>
void launch_attend_kernel(const AttnK& a, int hb, int qb, dim3 grid, hipStream_t st) {
  // timing labels: selected-entry lists (CSA) and dense visible ranges (HCA) apart
  const char* name = LIST ? "attend_csa_kernel" : "attend_hca_kernel";
  if (LIST && qb > 1) {
    if (qb == 8) LCS_LAUNCH(name, (attend_kernel<LIST, F8, 4, false, (LIST ? 8 : 1)>), grid, dim3(256), 0, st, a);
    else if (qb == 4) LCS_LAUNCH(name, (attend_kernel<LIST, F8, 4, false, (LIST ? 4 : 1)>), grid, dim3(256), 0, st, a);
    else LCS_LAUNCH(name, (attend_kernel<LIST, F8, 4, false, (LIST ? 2 : 1)>), grid, dim3(256), 0, st, a);
    return;
  }
  const bool pad = a.H < 16 * hb * (hb == 2 ? a.halves : 1);   // some workgroup has padding-only head blocks
  if (hb == 2 && pad) LCS_LAUNCH(name, (attend_kernel<LIST, F8, 2, true>), grid, dim3(256), 0, st, a);
  else if (hb == 2) LCS_LAUNCH(name, (attend_kernel<LIST, F8, 2, false>), grid, dim3(256), 0, st, a);
  else if (pad) LCS_LAUNCH(name, (attend_kernel<LIST, F8, 4, true>), grid, dim3(256), 0, st, a);
  else LCS_LAUNCH(name, (attend_kernel<LIST, F8, 4, false>), grid, dim3(256), 0, st, a);
}

int launch_attend(const AttendArgs& x, int64_t max_keys, hipStream_t st) {
  const int R = x.B * x.Tq;
  AttnK a;
  a.q = x.q; a.gamma_q = x.gamma_q; a.kv = x.kv; a.kv_ld = x.kv_ld; a.topk = x.topk; a.k = x.k;
  a.n_cap = x.n_cap; a.m = x.m; a.win = x.win; a.win_ld = x.win_ld; a.ring_cap = x.ring_cap;
  a.window = x.window; a.sink = x.sink; a.q_pos = x.q_pos; a.rope_offset = x.rope_offset;
  a.Tq = x.Tq; a.H = x.H; a.scale_log2 = x.scale * kLog2e; a.eps = x.eps; a.rf = rope_freq(x.theta);
  a.out = x.out;
  AttendPlan p = attend_plan(R, x.H, max_keys, x.topk != nullptr);
  const int qb = attend_rows_per_block(x.B, x.Tq, x.H, x.kv_ld, x.topk != nullptr, x.append != nullptr);
  if (qb > 1) {                                  // row blocks: one split, every key of the block's rows
    p.hb = 4;
    p.halves = 1;
    p.nsplit = 1;
    p.keys_per_split = 1 << 30;
  }
  a.keys_per_split = p.keys_per_split;
  a.nsplit = p.nsplit;
  a.halves = p.halves;
  a.part_o = static_cast<uint16_t*>(x.ws);
  a.part_ml = reinterpret_cast<float*>(static_cast<char*>(x.ws) +
                                       al256((size_t)R * a.nsplit * x.H * kHeadDim * 2));
  // HB = 2 with two halves: a flat grid, 16 workgroups per 8 (row, split) numbers (the two halves 8
  // apart), padded to a multiple of 16 (the padding returns at once)
  a.R = R;
  const bool flat = p.hb == 2 && p.halves == 2;
  const dim3 grid = flat   ? dim3((unsigned)(16 * (((int64_t)R * a.nsplit + 7) / 8)), 1u)
                    : qb > 1 ? dim3(1u, (unsigned)(x.B * ((x.Tq + qb - 1) / qb)))
                             : dim3((unsigned)a.nsplit, (unsigned)R);
  a.kv8 = x.kv8; a.kv_scale = x.kv_scale; a.win8 = x.win8; a.win_scale = x.win_scale;
  const bool f8 = x.kv8 != nullptr;
  a.app_rows = 0;
  a.ap = DecodeAppendArgs{};                    // no append: never read (app_rows = 0)
  a.rf_ap = a.rf;
  dim3 grid_k = grid;
  if (x.append && !x.topk && !flat) {           // the append's workgroups in extra rows of the grid
    a.ap = *x.append;
    a.rf_ap = rope_freq(x.append->theta);
    a.app_rows = (x.append->B + a.nsplit - 1) / a.nsplit;
    grid_k.y += (unsigned)a.app_rows;
  }
  if (x.append && a.app_rows == 0 && launch_decode_append(*x.append, st)) return 4;   // other shapes: first
  if (x.topk) {
    if (f8) launch_attend_kernel<true, true>(a, p.hb, qb, grid_k, st);
    else launch_attend_kernel<true, false>(a, p.hb, qb, grid_k, st);
  } else {
    if (f8) launch_attend_kernel<false, true>(a, p.hb, 1, grid_k, st);
    else launch_attend_kernel<false, false>(a, p.hb, 1, grid_k, st);
  }
  if (a.nsplit > 1) {
    const int64_t waves = (int64_t)R * x.H;
    const dim3 gm((unsigned)((waves + kMergeWaves - 1) / kMergeWaves)), bm(kMergeWaves * kWave);
    if (a.nsplit <= 4) LCS_LAUNCH("attend_merge_kernel", merge_kernel<4>, gm, bm, 0, st, a.part_o, a.part_ml, R, a.nsplit, x.H, x.sink, x.out);
    else if (a.nsplit <= 8) LCS_LAUNCH("attend_merge_kernel", merge_kernel<8>, gm, bm, 0, st, a.part_o, a.part_ml, R, a.nsplit, x.H, x.sink, x.out);
    else LCS_LAUNCH("attend_merge_kernel", merge_kernel<16>, gm, bm, 0, st, a.part_o, a.part_ml, R, a.nsplit, x.H, x.sink, x.out);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
