// Lightning-indexer scoring and per-query top-k block selection (page 1, "hybrid attention",
// CSA step 2; page 4 section 3.1: 64 indexer heads of dim 128, top-k 512; page 1: top-k 1024 at
// 1M context).  Score of entry s for the query at token t:  I_s = sum_h w_h * max(0, q_h . k_s),
// over the entries visible to t (s < t / m).  The min(k, n_vis) largest are kept, ties going to
// the lower index, and written ascending with -1 padding.
//
// Scoring is a dense contraction (query heads x entries x d_I) and runs on the matrix cores:
// E4M3FN codes on the gfx950 scaled fp8 MFMA (16x16x128, unit scales), or bf16 MFMA (16x16x32).
// Query rows are quantised in-kernel (absmax/448 per head row, RNE), their scales folded into the
// head weights, the key scale applied after the head sum (relu commutes with a positive scale).
//
// Selection is an exact radix select on the order-preserving uint32 image of the fp32 scores,
// extended by the complemented entry index so that every key is distinct:
//   decode (few query rows):  score kernel also histograms the top 11 bits of every score
//       (LDS, then integer atomics to a per-row global histogram) -> filter kernel, many
//       workgroups per row, appends entries of bins above the k-th's bin to the result and those of
//       its bin to a candidate list -> final kernel, one workgroup per row, resolves the
//       candidates digit by digit, sorts the result ascending and writes it out.
//   prefill (many query rows): one workgroup per row does histogram, filter and the same final.
#include <limits.h>

#include <type_traits>

#include "common.h"
#include "kernels.h"

namespace lcs {

namespace {

constexpr int kBins = 2048;                 // top 11 bits of the score key
constexpr int kBinShift = 21;
constexpr int kHistRow = 2 * kBins + 4;     // per row: level-1 bins, level-2 bins (candidates' next 11 bits), spare
constexpr int kScoreChunk = 1024;           // entries per scoring workgroup
constexpr int kFilterChunk = 4096;          // entries per filter workgroup
constexpr int kSelThreads = 256;
constexpr int kMaxTopk = 2048;

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

struct Ws {
  float* scores;                  // [R, nsp]
  uint32_t* hist;                 // [R, kHistRow]: histograms of the top score-key bits, then of the next 11
  unsigned long long* comb;       // [R, nsp]: kept entries per chunk (decode) / candidates (prefill)
  uint2* counts;                  // [R, nchunk]: per decode chunk (kept, above the threshold bin)
  int64_t nsp;
  int nchunk;
};

inline int64_t n_chunks(int64_t n_cap) { return (n_cap + kFilterChunk - 1) / kFilterChunk; }

Ws carve(void* ws, int R, int64_t n_cap) {
  Ws w;
  w.nsp = (n_cap + 63) & ~(int64_t)63;
  w.nchunk = (int)n_chunks(n_cap);
  char* p = static_cast<char*>(ws);
  w.scores = reinterpret_cast<float*>(p);
  p += al256((size_t)R * w.nsp * 4);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)R * kHistRow * 4);
  w.comb = reinterpret_cast<unsigned long long*>(p);
  p += al256((size_t)R * w.nsp * 8);
  w.counts = reinterpret_cast<uint2*>(p);
  return w;
}

__device__ __forceinline__ int64_t n_visible(const int64_t* q_pos, int64_t r, int m, int64_t n_cap) {
  int64_t t = q_pos[r];
  int64_t n = t >= 0 ? t / m : 0;
  return n < n_cap ? n : n_cap;
}

// ------------------------------------------------------------------------------------ clear
__global__ void clear_u32_kernel(uint32_t* __restrict__ p, int64_t n) {
  for (int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; i < n; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0u;
}

// ------------------------------------------------------------------------------------ scoring
// Workgroup: 4 waves.  QW = query rows per wave.  QW == 1: one query per workgroup, the waves split
// the chunk's entries (decode).  QW == 4: 16 queries per workgroup, every wave scores the whole
// chunk for its 4 queries (prefill; entries are re-read from L1/L2, not HBM).
template <bool FP8, int KS, int HBI, int QW>
__global__ void __launch_bounds__(256)
index_score_kernel(const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w_idx,
                   const void* __restrict__ ik, const float* __restrict__ ik_scale, int64_t ik_ld,
                   const int64_t* __restrict__ q_pos, int64_t n_cap, int Tq, int H_I, int dI, int m,
                   float* __restrict__ scores, uint32_t* __restrict__ hist, int64_t nsp) {
  constexpr int QWAVES = QW == 1 ? 1 : 4;       // waves that split the queries
  constexpr int QTILE = QW * QWAVES;
  constexpr bool HIST = (QW == 1);
  __shared__ uint32_t lhist[HIST ? kBins : 1];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int tiles_per_b = (Tq + QTILE - 1) / QTILE;
  const int b = blockIdx.y / tiles_per_b;
  const int tq0 = (blockIdx.y % tiles_per_b) * QTILE;
  const int64_t c0 = (int64_t)blockIdx.x * kScoreChunk;

  // entry limit of this workgroup = max n_vis over its queries
  int64_t nv_max = 0;
  for (int i = 0; i < QTILE; ++i) {
    const int tq = tq0 + i;
    if (tq < Tq) {
      const int64_t nv = n_visible(q_pos, (int64_t)b * Tq + tq, m, n_cap);
      nv_max = nv > nv_max ? nv : nv_max;
    }
  }
  if (c0 >= nv_max) return;                    // uniform across the workgroup

  if (HIST) {
    for (int i = threadIdx.x; i < kBins; i += 256) lhist[i] = 0u;
    __syncthreads();
  }

  // ---- per-query operands: A fragments (head rows) and folded head weights ----
  const int qgroup = wave % QWAVES;
  const int kpart = wave / QWAVES;
  constexpr int KWAVES = 4 / QWAVES;
  typedef typename std::conditional<FP8, intx8, uint4>::type AFrag;
  AFrag afr[QW][HBI][KS];
  float wq[QW][HBI][4];
  int64_t nvis[QW];
  int64_t rowq[QW];
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    const int tq = tq0 + qgroup * QW + qw;
    const bool qvalid = tq < Tq;
    const int64_t r = (int64_t)b * Tq + (qvalid ? tq : 0);
    rowq[qw] = r;
    nvis[qw] = qvalid ? n_visible(q_pos, r, m, n_cap) : 0;
#pragma unroll
    for (int hb = 0; hb < HBI; ++hb) {
      const int head = hb * 16 + c16;
      const bool hv = qvalid && head < H_I;
      const uint16_t* qrow = q_idx + (r * H_I + (hv ? head : 0)) * dI;
      float wh = hv ? bf2f(w_idx[r * H_I + head]) : 0.f;
      if (FP8) {
        // dims [32g, 32g+32) of this head row
        uint4 raw[4];
#pragma unroll
        for (int u = 0; u < 4; ++u)
          raw[u] = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * g + 8 * u) : make_uint4(0, 0, 0, 0);
        float v[32];
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          v[8 * u + 0] = bf2f_lo(raw[u].x); v[8 * u + 1] = bf2f_hi(raw[u].x);
          v[8 * u + 2] = bf2f_lo(raw[u].y); v[8 * u + 3] = bf2f_hi(raw[u].y);
          v[8 * u + 4] = bf2f_lo(raw[u].z); v[8 * u + 5] = bf2f_hi(raw[u].z);
          v[8 * u + 6] = bf2f_lo(raw[u].w); v[8 * u + 7] = bf2f_hi(raw[u].w);
        }
        float amax = 0.f;
#pragma unroll
        for (int j = 0; j < 32; ++j) amax = fmaxf(amax, fabsf(v[j]));
        amax = max_rows4(amax);
        const float s = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
        intx8 codes;
#pragma unroll
        for (int j = 0; j < 8; ++j) {
          const uint32_t b0 = f2e4m3(__fdiv_rn(v[4 * j + 0], s));
          const uint32_t b1 = f2e4m3(__fdiv_rn(v[4 * j + 1], s));
          const uint32_t b2 = f2e4m3(__fdiv_rn(v[4 * j + 2], s));
          const uint32_t b3 = f2e4m3(__fdiv_rn(v[4 * j + 3], s));
          codes[j] = (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
        }
        if (!hv) codes = intx8{0, 0, 0, 0, 0, 0, 0, 0};
        afr[qw][hb][0] = *reinterpret_cast<AFrag*>(&codes);
        wh *= s;
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 a = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
          afr[qw][hb][ks] = *reinterpret_cast<AFrag*>(&a);
        }
      }
      // the D fragment of this lane holds heads 16hb + 4g + i: fetch their weights
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[qw][hb][i] = __shfl(wh, 4 * g + i, kWave);
    }
  }

  // ---- entry loop ----
  const int64_t span = kScoreChunk / KWAVES;
  int64_t e_lo = c0 + kpart * span;
  int64_t e_hi = e_lo + span;
  if (e_hi > nv_max) e_hi = nv_max;
  const uint8_t* ik8 = static_cast<const uint8_t*>(ik) + (int64_t)b * ik_ld * dI;
  const uint16_t* ik16 = static_cast<const uint16_t*>(ik) + (int64_t)b * ik_ld * dI;
  const float* ksc = ik_scale ? ik_scale + (int64_t)b * ik_ld : nullptr;

  for (int64_t e0 = e_lo; e0 < e_hi; e0 += 64) {
    typedef typename std::conditional<FP8, intx8, uint4>::type BFrag;
    BFrag bfr[4][KS];
    float kscale[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = e0 + 16 * u + c16;
      const bool ev = e < e_hi;
      if (FP8) {
        intx8 v = intx8{0, 0, 0, 0, 0, 0, 0, 0};
        if (ev) {
          const uint4* p = reinterpret_cast<const uint4*>(ik8 + e * 128 + 32 * g);
          const uint4 x0 = p[0], x1 = p[1];
          v = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        }
        bfr[u][0] = *reinterpret_cast<BFrag*>(&v);
        kscale[u] = ev ? ksc[e] : 0.f;
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 v = ev ? *reinterpret_cast<const uint4*>(ik16 + e * dI + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
          bfr[u][ks] = *reinterpret_cast<BFrag*>(&v);
        }
        kscale[u] = 1.f;
      }
    }
#pragma unroll
    for (int qw = 0; qw < QW; ++qw) {
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        float part = 0.f;
#pragma unroll
        for (int hb = 0; hb < HBI; ++hb) {
          floatx4 acc = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
          for (int ks = 0; ks < KS; ++ks) {
            if (FP8)
              acc = mfma_fp8(*reinterpret_cast<intx8*>(&afr[qw][hb][ks]), *reinterpret_cast<intx8*>(&bfr[u][ks]), acc);
            else
              acc = mfma_bf16(*reinterpret_cast<uint4*>(&afr[qw][hb][ks]), *reinterpret_cast<uint4*>(&bfr[u][ks]), acc);
          }
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wq[qw][hb][i] * fmaxf(acc[i], 0.f);
        }
        part = sum_rows4(part);
        const int64_t e = e0 + 16 * u + c16;
        if (g == 0 && e < nvis[qw]) {
          const float sc = part * kscale[u] + 0.0f;
          scores[rowq[qw] * nsp + e] = sc;
          if (HIST) atomicAdd(&lhist[float_key(sc) >> kBinShift], 1u);
        }
      }
    }
  }

  if (HIST) {
    __syncthreads();
    uint32_t* gh = hist + rowq[0] * kHistRow;
    for (int i = threadIdx.x; i < kBins; i += 256) {
      const uint32_t v = lhist[i];
      if (v) atomicAdd(gh + i, v);
    }
  }
}

// Decode scoring: one query row per workgroup, `chunk` entries per workgroup.  The 4 waves quantise
// one 16-head block each into LDS (codes + folded weights), then stream the chunk in 64-entry groups
// interleaved across waves, with the next group's loads in flight while the current group's 4*HBI
// MFMAs run back to back; the epilogue applies relu and the head weights and histograms the scores.
template <bool FP8, int KS, int HBI>
__global__ void __launch_bounds__(256, (FP8 || KS * HBI <= 8) ? 2 : 1)
index_score_decode_kernel(const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w_idx,
                          const void* __restrict__ ik, const float* __restrict__ ik_scale, int64_t ik_ld,
                          const int64_t* __restrict__ q_pos, int64_t n_cap, int Tq, int H_I, int dI, int m,
                          int64_t chunk, float* __restrict__ scores, uint32_t* __restrict__ hist, int64_t nsp) {
  typedef typename std::conditional<FP8, intx8, uint4>::type Frag;
  __shared__ uint32_t lhist[kBins];
  __shared__ Frag s_afr[HBI][KS][kWave];
  __shared__ float s_w[HBI * 16];

  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t r = blockIdx.y;
  const int64_t b = r / Tq;
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const int64_t c0 = (int64_t)blockIdx.x * chunk;
  if (c0 >= nv) return;                                  // uniform
  const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;

  for (int i = threadIdx.x; i < kBins; i += 256) lhist[i] = 0u;
  if (wave < HBI) {
    const int head = wave * 16 + c16;
    const bool hv = head < H_I;
    const int hl = hv ? head : H_I - 1;
    const uint16_t* qrow = q_idx + (r * H_I + hl) * dI;
    float wh = bf2f(w_idx[r * H_I + hl]);
    if (!hv) wh = 0.f;
    if (FP8) {
      uint4 raw[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const uint4*>(qrow + 32 * g + 8 * u);
      float amax = 0.f;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf2f_lo(wd[j])), fabsf(bf2f_hi(wd[j]))));
      }
      amax = max_rows4(amax);
      const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
      intx8 codes;
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
        for (int j = 0; j < 2; ++j) {
          const uint32_t b0 = f2e4m3(__fdiv_rn(bf2f_lo(wd[2 * j]), sc));
          const uint32_t b1 = f2e4m3(__fdiv_rn(bf2f_hi(wd[2 * j]), sc));
          const uint32_t b2 = f2e4m3(__fdiv_rn(bf2f_lo(wd[2 * j + 1]), sc));
          const uint32_t b3 = f2e4m3(__fdiv_rn(bf2f_hi(wd[2 * j + 1]), sc));
          codes[2 * u + j] = (int)(b0 | (b1 << 8) | (b2 << 16) | (b3 << 24));
        }
      }
      if (!hv) codes = intx8{0, 0, 0, 0, 0, 0, 0, 0};
      s_afr[wave][0][lane] = *reinterpret_cast<Frag*>(&codes);
      wh *= sc;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        uint4 a = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
        if (!hv) a = make_uint4(0, 0, 0, 0);
        s_afr[wave][ks][lane] = *reinterpret_cast<Frag*>(&a);
      }
    }
    if (g == 0) s_w[wave * 16 + c16] = wh;
  }
  __syncthreads();
  Frag afr[HBI][KS];
  float wq[HBI][4];
#pragma unroll
  for (int hb = 0; hb < HBI; ++hb) {
#pragma unroll
    for (int ks = 0; ks < KS; ++ks) afr[hb][ks] = s_afr[hb][ks][lane];
#pragma unroll
    for (int i = 0; i < 4; ++i) wq[hb][i] = s_w[hb * 16 + 4 * g + i];
  }

  const uint8_t* ik8 = static_cast<const uint8_t*>(ik) + b * ik_ld * dI;
  const uint16_t* ik16 = static_cast<const uint16_t*>(ik) + b * ik_ld * dI;
  const float* ksc = ik_scale ? ik_scale + b * ik_ld : nullptr;
  float* srow = scores + r * nsp;
  const int64_t ngroups = (c1 - c0 + 63) / 64;

  Frag cur[4][KS], nxt[4][KS], nx2[4][KS];
  float cs, ns, n2;
  // Loads are unconditional (entry index clamped into the chunk) so that the compiler keeps them in
  // flight; out-of-range entries are zeroed by a select and never stored.  One scale load per group:
  // lane l takes entry 64 gi + l (row-group u of the fragments needs lanes 16u .. 16u+15).
  auto load_group = [&](int64_t gi, Frag (&fr)[4][KS], float& sc) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t e = c0 + 64 * gi + 16 * u + c16;
      e = e < c1 ? e : c1 - 1;
      if (FP8) {
        const uint4* p = reinterpret_cast<const uint4*>(ik8 + e * 128 + 32 * g);
        const uint4 x0 = p[0], x1 = p[1];
        intx8 v = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
        fr[u][0] = *reinterpret_cast<Frag*>(&v);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 v = *reinterpret_cast<const uint4*>(ik16 + e * dI + 32 * ks + 8 * g);
          fr[u][ks] = *reinterpret_cast<Frag*>(&v);
        }
      }
    }
    if (FP8) {
      int64_t e = c0 + 64 * gi + lane;
      sc = ksc[e < c1 ? e : c1 - 1];        // clamped entries are never stored
    } else {
      sc = 1.f;
    }
  };

  // Groups of this wave: wave + 4t, t = 0 .. nt-1.  Three register buffers rotate by unrolling (a
  // copy between buffers would wait for the loads in flight); two groups stay in flight ahead of the
  // one being computed.  Loads past the end re-read the last group (never computed).
  const int64_t nt = ngroups > wave ? (ngroups - wave + 3) / 4 : 0;
  auto gidx = [&](int64_t t) -> int64_t { return wave + 4 * (t < nt ? t : nt - 1); };
  auto compute_group = [&](const Frag (&fr)[4][KS], float sc_lane, int64_t gi) {
    // every row group's scales in every lane (same column): rows 0..3 = entries 16u + c16
    float sc[4];
    {
      const auto p16 = __builtin_amdgcn_permlane16_swap(__float_as_uint(sc_lane), __float_as_uint(sc_lane), false, false);
      const auto lo = __builtin_amdgcn_permlane32_swap(p16[0], p16[0], false, false);   // rows 0, 2
      const auto hi = __builtin_amdgcn_permlane32_swap(p16[1], p16[1], false, false);   // rows 1, 3
      sc[0] = __uint_as_float(lo[0]); sc[1] = __uint_as_float(hi[0]);
      sc[2] = __uint_as_float(lo[1]); sc[3] = __uint_as_float(hi[1]);
    }
    floatx4 acc[4][HBI];
#pragma unroll
    for (int u = 0; u < 4; ++u)
#pragma unroll
      for (int hb = 0; hb < HBI; ++hb) {
        floatx4 a = {0.f, 0.f, 0.f, 0.f};
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          if (FP8)
            a = mfma_fp8(*reinterpret_cast<const intx8*>(&afr[hb][ks]), *reinterpret_cast<const intx8*>(&fr[u][ks]), a);
          else
            a = mfma_bf16(*reinterpret_cast<const uint4*>(&afr[hb][ks]), *reinterpret_cast<const uint4*>(&fr[u][ks]), a);
        }
        acc[u][hb] = a;
      }
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      float part = 0.f;
#pragma unroll
      for (int hb = 0; hb < HBI; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) part += wq[hb][i] * fmaxf(acc[u][hb][i], 0.f);
      part = sum_rows4(part);
      const int64_t e = c0 + 64 * gi + 16 * u + c16;
      if (g == 0 && e < c1) {
        const float v = part * sc[u] + 0.0f;
        srow[e] = v;
        atomicAdd(&lhist[float_key(v) >> kBinShift], 1u);
      }
    }
  };
  if (nt > 0) {
    load_group(gidx(0), cur, cs);
    load_group(gidx(1), nxt, ns);
    for (int64_t t = 0; t < nt; t += 3) {
      load_group(gidx(t + 2), nx2, n2);
      compute_group(cur, cs, gidx(t));
      if (t + 1 >= nt) break;
      load_group(gidx(t + 3), cur, cs);
      compute_group(nxt, ns, gidx(t + 1));
      if (t + 2 >= nt) break;
      load_group(gidx(t + 4), nxt, ns);
      compute_group(nx2, n2, gidx(t + 2));
    }
  }
  __syncthreads();
  uint32_t* gh = hist + r * kHistRow;
  for (int i = threadIdx.x; i < kBins; i += 256) {
    const uint32_t v = lhist[i];
    if (v) atomicAdd(gh + i, v);
  }
}

// ------------------------------------------------------------------------------------ selection
// Block-wide exclusive prefix sum over the 256 threads; *total receives the sum.  s_w: 4 words.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* s_w, uint32_t* total) {
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  uint32_t incl = v;
#pragma unroll
  for (int o = 1; o < kWave; o <<= 1) {
    const uint32_t t = __shfl_up(incl, o, kWave);
    if (lane >= o) incl += t;
  }
  if (lane == kWave - 1) s_w[wave] = incl;
  __syncthreads();
  uint32_t base = 0, tot = 0;
#pragma unroll
  for (int w = 0; w < kSelThreads / kWave; ++w) {
    const uint32_t x = s_w[w];
    base += w < wave ? x : 0u;
    tot += x;
  }
  __syncthreads();                                // s_w may be reused
  *total = tot;
  return base + incl - v;
}

// Threshold bin from a complete 2048-bin histogram: the bin T holding the k-th largest score and
// the number of scores in bins above it.  256 threads, 8 bins each; T stays as initialised (-1: keep
// everything) when the histogram holds fewer than k scores.
// (the thread's 8 bins, tid*8 .. tid*8+7, already loaded)
__device__ __forceinline__ void find_threshold_bins(const uint32_t (&loc)[8], int k, int* T_out, int* above_out,
                                                    uint32_t* s_w) {
  const int tid = threadIdx.x;
  uint32_t sum = 0;
#pragma unroll
  for (int j = 0; j < 8; ++j) sum += loc[j];
  uint32_t total;
  const uint32_t below = block_excl_scan(sum, s_w, &total);   // bins under this thread's range
  const uint32_t higher = total - below - sum;                 // bins above it
  if (higher < (uint32_t)k && higher + sum >= (uint32_t)k) {
    uint32_t cum = higher;
    for (int j = 7; j >= 0; --j) {
      if (cum + loc[j] >= (uint32_t)k) { *T_out = tid * 8 + j; *above_out = (int)cum; break; }
      cum += loc[j];
    }
  }
  __syncthreads();
}

__device__ __forceinline__ void find_threshold(const uint32_t* h, int k, int* T_out, int* above_out, uint32_t* s_w) {
  const uint4 a = *reinterpret_cast<const uint4*>(h + threadIdx.x * 8);
  const uint4 b = *reinterpret_cast<const uint4*>(h + threadIdx.x * 8 + 4);
  const uint32_t loc[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
  find_threshold_bins(loc, k, T_out, above_out, s_w);
}

// 53-bit candidate key: the 21 score-key bits below the bin, then the complemented entry index, so
// that larger score wins and, among equal scores, the lower index wins; every key is distinct.
__device__ __forceinline__ unsigned long long cand_key(uint32_t key32, int32_t s) {
  return ((unsigned long long)(key32 & 0x1FFFFFu) << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)s);
}
constexpr unsigned long long kAbove = 1ull << 63;   // kept entry from a bin above the threshold bin

// Decode selection, per row.  The kept entries of the row's chunks, concatenated in chunk
// order, are the row's candidates in index order.  The filter's second histogram (the next 11 key
// bits of the threshold-bin entries) usually pins the k-th winner's key; otherwise digit passes over
// the remaining key bits finish the job.  The winners are written in list order, so the result is
// ascending without a sort.  Up to kFinalCache kept entries are staged in LDS (thread t owns list
// positions 16t .. 16t+15, stored transposed so that both the staging writes and the per-thread
// reads are free of bank conflicts); beyond that every pass reads the list from global memory.
constexpr int kFinalCache = 4096;
constexpr int kFinalSeg = kFinalCache / kSelThreads;        // 16 list positions per thread
constexpr int kFinalStride = kSelThreads + 1;               // LDS row stride of the transposed list
constexpr int kMaxDecodeChunks = 2048;                      // rows up to 8M entries take this path

__device__ __forceinline__ int final_slot(int i) { return (i % kFinalSeg) * kFinalStride + i / kFinalSeg; }

struct FinalShared {
  unsigned long long list[kFinalSeg * kFinalStride];
  uint32_t keep[kMaxDecodeChunks];   // kept entries per chunk
  uint32_t pos[kMaxDecodeChunks];    // their offset in the concatenated list / in the output
  uint32_t h[256];
  unsigned long long prefix;
  int remaining, done, shift, T2, above2;
};

// Row r's selection (nv visible entries).
__device__ __forceinline__ void final_select(FinalShared& sh, uint32_t* s_w, int64_t r, int64_t nv,
                                             const unsigned long long* __restrict__ comb,
                                             const uint2* __restrict__ counts, const uint32_t* __restrict__ hist,
                                             int64_t nsp, int nchunk, int k, const float* __restrict__ scores,
                                             int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  auto& s_list = sh.list;
  auto& s_keep = sh.keep;
  auto& s_pos = sh.pos;
  auto& s_h = sh.h;
  auto& s_prefix = sh.prefix;
  auto& s_remaining = sh.remaining;
  auto& s_done = sh.done;
  auto& s_shift = sh.shift;
  auto& s_T2 = sh.T2;
  auto& s_above2 = sh.above2;
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  constexpr int kWaves = kSelThreads / kWave;
  int32_t* out = topk_idx + r * k;
  float* out_s = topk_score ? topk_score + r * k : nullptr;
  const float* srow = scores + r * nsp;
  if (nv <= k) {                                    // every visible entry, ascending
    for (int64_t i = tid; i < k; i += kSelThreads) {
      out[i] = i < nv ? (int32_t)i : -1;
      if (out_s) out_s[i] = i < nv ? srow[i] : -INFINITY;
    }
    return;
  }
  const int nch = (int)((nv + kFilterChunk - 1) / kFilterChunk);
  const unsigned long long* lrow = comb + r * nsp;

  // ---- one round trip: the per-chunk counts and, speculatively, the first 64 list entries of each
  //      of the first 64 chunks (wave w: chunks w, w + 4, ...), which usually hold the whole list ----
  constexpr int kHeadChunks = kWaves * 16;
  const bool heads = nch <= kHeadChunks;
  unsigned long long vh[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int c = min(wave + kWaves * u, nch - 1);
    vh[u] = lrow[min((int64_t)c * kFilterChunk + lane, nv - 1)];
  }
  const uint32_t* h2 = hist + r * kHistRow + kBins;
  const uint4 h2a = *reinterpret_cast<const uint4*>(h2 + tid * 8);
  const uint4 h2b = *reinterpret_cast<const uint4*>(h2 + tid * 8 + 4);
  constexpr int kPerT = kMaxDecodeChunks / kSelThreads;   // 8
  uint32_t kc[kPerT];
  uint32_t ksum = 0, asum = 0;
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = tid * kPerT + u;
    const uint2 cc = counts[r * nchunk + (c < nch ? c : 0)];
    kc[u] = c < nch ? cc.x : 0u;
    ksum += kc[u];
    asum += c < nch ? cc.y : 0u;
  }
  uint32_t total_keep, total_above;
  uint32_t off = block_excl_scan(ksum, s_w, &total_keep);
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = tid * kPerT + u;
    s_keep[c] = kc[u];
    s_pos[c] = off;
    off += kc[u];
  }
  block_excl_scan(asum, s_w, &total_above);       // (its barriers also publish s_keep / s_pos)
  const int need = k - (int)total_above;          // winners among the threshold-bin entries (>= 1)
  const bool cached = total_keep <= (uint32_t)kFinalCache;

  // ---- stage the list: wave w copies chunks w, w + 4, ...; sixteen chunks' loads in flight ----
  if (cached && heads) {
    // the 16 chunks' counts and offsets first (all LDS reads in flight together), then the stores
    int nk[16], pk[16];
#pragma unroll
    for (int u = 0; u < 16; ++u) {
      const int c = wave + kWaves * u;
      const int cc = c < nch ? c : nch - 1;
      nk[u] = c < nch ? (int)s_keep[cc] : 0;
      pk[u] = (int)s_pos[cc];
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (lane < nk[u]) s_list[final_slot(pk[u] + lane)] = vh[u];
#pragma unroll
    for (int u = 0; u < 16; ++u)                    // chunks with more than 64 kept entries
      for (int j = kWave + lane; j < nk[u]; j += kWave)
        s_list[final_slot(pk[u] + j)] = lrow[(int64_t)(wave + kWaves * u) * kFilterChunk + j];
  }
  if (cached && !heads) {
    for (int cb = wave; cb < nch; cb += kWaves * 16) {
      unsigned long long v[16];
      int n[16];
#pragma unroll
      for (int u = 0; u < 16; ++u) {               // in-range chunk, unconditional load (no branches)
        const int c = min(cb + kWaves * u, nch - 1);
        n[u] = (int)s_keep[c];
        v[u] = lrow[(int64_t)c * kFilterChunk + min(lane, max(n[u] - 1, 0))];
      }
#pragma unroll
      for (int u = 0; u < 16; ++u) {
        const int c = cb + kWaves * u;
        if (c < nch && lane < n[u]) s_list[final_slot((int)s_pos[c] + lane)] = v[u];
      }
    }
  }
  if (cached && !heads) {
    for (int c = wave; c < nch; c += kWaves)        // chunks with more than 64 kept entries
      for (int j = kWave + lane; j < (int)s_keep[c]; j += kWave)
        s_list[final_slot((int)s_pos[c] + j)] = lrow[(int64_t)c * kFilterChunk + j];
  }

  // ---- level-2 threshold: the bin of the next 11 key bits that holds the need-th winner ----
  if (tid == 0) { s_T2 = 0; s_above2 = 0; }
  __syncthreads();
  {
    const uint32_t loc[8] = {h2a.x, h2a.y, h2a.z, h2a.w, h2b.x, h2b.y, h2b.z, h2b.w};
    find_threshold_bins(loc, need, &s_T2, &s_above2, s_w);
    if (tid == s_T2 / 8) {                          // the thread holding bin T2
      const int rem = need - s_above2;
      s_remaining = rem;
      s_prefix = (unsigned long long)s_T2;
      s_shift = 42;                                 // candidates' keys >> 42 = their level-2 bin
      s_done = loc[s_T2 % 8] == (uint32_t)rem ? 1 : 0;
    }
  }
  __syncthreads();

  // visit every kept entry once: the LDS copy (thread t: positions 16t..16t+15), or chunk by chunk
  // from global memory
  auto for_each = [&](auto&& f) {
    if (cached) {
#pragma unroll
      for (int u = 0; u < kFinalSeg; ++u)
        if (tid * kFinalSeg + u < (int)total_keep) f(s_list[u * kFinalStride + tid]);
    } else {
      for (int c = wave; c < nch; c += kWaves)
        for (int j = lane; j < (int)s_keep[c]; j += kWave) f(lrow[(int64_t)c * kFilterChunk + j]);
    }
  };

  // ---- digit passes over the rest of the key (10 score bits, then the complemented index) ----
  if (!s_done) {
    int shift = 42;
    for (int pass = 0; pass < 6; ++pass) {
      const int width = shift >= 8 ? 8 : shift;
      shift -= width;
      s_h[tid] = 0u;
      __syncthreads();
      const unsigned long long pre = s_prefix;
      const uint32_t dmask = (1u << width) - 1u;
      for_each([&](unsigned long long e) {
        if (!(e & kAbove) && (e >> (shift + width)) == pre) atomicAdd(&s_h[(uint32_t)(e >> shift) & dmask], 1u);
      });
      __syncthreads();
      if (tid < kWave) {
        // lane j covers digits 255-4j .. 252-4j (top first)
        uint32_t c[4];
        uint32_t lsum = 0;
#pragma unroll
        for (int u = 0; u < 4; ++u) { c[u] = s_h[255 - 4 * tid - u]; lsum += c[u]; }
        uint32_t incl = lsum;
#pragma unroll
        for (int o = 1; o < kWave; o <<= 1) {
          const uint32_t v = __shfl_up(incl, o, kWave);
          if (tid >= o) incl += v;
        }
        const uint32_t rem = (uint32_t)s_remaining;
        const uint64_t hit = __ballot(incl >= rem);
        const int first = __ffsll((unsigned long long)hit) - 1;
        if (tid == first) {
          uint32_t cum = incl - lsum;
          for (int u = 0; u < 4; ++u) {
            if (cum + c[u] >= rem) {
              const uint32_t d = 255u - 4u * tid - u;
              const uint32_t left = rem - cum;
              s_remaining = (int)left;
              s_prefix = (s_prefix << width) | d;
              s_shift = shift;
              if (c[u] == left || shift == 0) s_done = 1;
              break;
            }
            cum += c[u];
          }
        }
      }
      __syncthreads();
      if (s_done) break;
    }
  }
  const unsigned long long thr = s_prefix;
  const int ts = s_shift;
  auto wins = [&](unsigned long long e) { return (e & kAbove) || (e >> ts) >= thr; };
  auto index_of = [](unsigned long long e) { return (int32_t)(0xFFFFFFFFu - (uint32_t)e); };

  // ---- winners in list order = ascending index ----
  if (cached) {
    unsigned long long ev[kFinalSeg];
    uint32_t win = 0;
#pragma unroll
    for (int u = 0; u < kFinalSeg; ++u) {
      ev[u] = s_list[u * kFinalStride + tid];
      if (tid * kFinalSeg + u < (int)total_keep && wins(ev[u])) win |= 1u << u;
    }
    uint32_t tot;
    uint32_t pos = block_excl_scan((uint32_t)__popc(win), s_w, &tot);
#pragma unroll
    for (int u = 0; u < kFinalSeg; ++u) {
      if (((win >> u) & 1u) && pos < (uint32_t)k) {   // exactly k winners; the bound is a guard
        const int32_t e = index_of(ev[u]);
        out[pos] = e;
        if (out_s) out_s[pos] = srow[e];
        ++pos;
      }
    }
    // every slot is written: with consistent inputs tot == k; the -1 fill is a guard
    for (int i = (int)tot + tid; i < k; i += kSelThreads) {
      out[i] = -1;
      if (out_s) out_s[i] = -INFINITY;
    }
  } else {
    // winners per chunk, their output offsets, then each wave writes its chunks in order
    for (int c = wave; c < nch; c += kWaves) {
      uint32_t n = 0;
      for (int j = lane; j < (int)s_keep[c]; j += kWave) n += wins(lrow[(int64_t)c * kFilterChunk + j]) ? 1u : 0u;
      n = (uint32_t)wave_sum((float)n);                     // exact: counts <= 4096
      if (lane == 0) s_keep[c] = n;
    }
    __syncthreads();
    uint32_t wsum = 0;
    uint32_t wc[kPerT];
#pragma unroll
    for (int u = 0; u < kPerT; ++u) {
      const int c = tid * kPerT + u;
      wc[u] = c < nch ? s_keep[c] : 0u;
      wsum += wc[u];
    }
    uint32_t tot;
    uint32_t o2 = block_excl_scan(wsum, s_w, &tot);
    for (int i = (int)tot + tid; i < k; i += kSelThreads) {   // guard, as in the cached path
      out[i] = -1;
      if (out_s) out_s[i] = -INFINITY;
    }
#pragma unroll
    for (int u = 0; u < kPerT; ++u) { s_pos[tid * kPerT + u] = o2; o2 += wc[u]; }
    __syncthreads();
    for (int c = wave; c < nch; c += kWaves) {
      uint32_t base = s_pos[c];
      const int nk = (int)counts[r * nchunk + c].x;        // the chunk's list length
      for (int j0 = 0; j0 < nk; j0 += kWave) {
        const int j = j0 + lane;
        const unsigned long long e = lrow[(int64_t)c * kFilterChunk + (j < nk ? j : 0)];
        const bool wv = j < nk && wins(e);
        const uint64_t bal = __ballot(wv);
        const uint32_t p = base + (uint32_t)__popcll(bal & ((1ull << lane) - 1ull));
        if (wv && p < (uint32_t)k) {
          const int32_t ix = index_of(e);
          out[p] = ix;
          if (out_s) out_s[p] = srow[ix];
        }
        base += (uint32_t)__popcll(bal);
      }
    }
  }
}

// Decode filter: one workgroup per chunk of kFilterChunk entries of a row.  The entries whose bin is
// above the threshold bin or equal to it are written, in index order, at the start of the chunk's
// own region of the row's list (value: above flag | 53-bit key), with the chunk's counts and the
// second-level histogram of the threshold-bin entries.  The output order does not depend on
// scheduling.  (Handing the selection to the last workgroup of a row would need device-scope fences,
// i.e. an L2 write-back per workgroup, which costs far more than the kernel boundary.)
__global__ void __launch_bounds__(kSelThreads)
topk_filter_kernel(const float* __restrict__ scores, uint32_t* __restrict__ hist,
                   unsigned long long* __restrict__ comb, uint2* __restrict__ counts, int64_t nsp, int nchunk,
                   const int64_t* __restrict__ q_pos, int m, int64_t n_cap, int k) {
  __shared__ uint32_t s_w[kSelThreads / kWave];
  __shared__ int sT, sAbove;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.y;
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const int64_t c0 = (int64_t)blockIdx.x * kFilterChunk;
  if (c0 >= nv) return;                                      // uniform
  constexpr int kPer = kFilterChunk / kSelThreads;           // 16 consecutive entries per thread
  const int64_t e0 = c0 + (int64_t)kPer * tid;
  const float* srow = scores + r * nsp;
  const int64_t q4max = (nv - 1) >> 2;                       // last readable float4 (nsp is a multiple of 64)
  uint32_t keys[kPer];
#pragma unroll
  for (int q = 0; q < kPer / 4; ++q) {                       // clamped, unconditional loads
    const int64_t q4 = (e0 >> 2) + q;
    const float4 x = *reinterpret_cast<const float4*>(srow + 4 * (q4 < q4max ? q4 : q4max));
    keys[4 * q + 0] = float_key(x.x);
    keys[4 * q + 1] = float_key(x.y);
    keys[4 * q + 2] = float_key(x.z);
    keys[4 * q + 3] = float_key(x.w);
  }
  if (tid == 0) { sT = -1; sAbove = 0; }
  __syncthreads();
  if (nv > k) find_threshold(hist + r * kHistRow, k, &sT, &sAbove, s_w);
  const int T = sT;
  uint32_t keep = 0, above = 0;
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    const bool valid = e0 + i < nv;
    const int bin = (int)(keys[i] >> kBinShift);
    keep |= (valid && bin >= T ? 1u : 0u) << i;
    above |= (valid && bin > T ? 1u : 0u) << i;
  }
  const uint32_t packed = (uint32_t)__popc(keep) | ((uint32_t)__popc(above) << 16);   // <= 4096 each
  uint32_t total;
  const uint32_t base = block_excl_scan(packed, s_w, &total);
  uint32_t pos = base & 0xFFFFu;
  unsigned long long* out = comb + r * nsp + c0;
  uint32_t* h2 = hist + r * kHistRow + kBins;   // level 2: candidates' next 11 bits
#pragma unroll
  for (int i = 0; i < kPer; ++i) {
    if ((keep >> i) & 1u) {
      const bool ab = (above >> i) & 1u;
      out[pos] = (ab ? kAbove : 0ull) | cand_key(keys[i], (int32_t)(e0 + i));
      if (!ab) atomicAdd(&h2[(keys[i] >> (kBinShift - 11)) & (kBins - 1)], 1u);
      ++pos;
    }
  }
  if (tid == 0) counts[r * nchunk + blockIdx.x] = make_uint2(total & 0xFFFFu, total >> 16);
}

// Decode final: one workgroup per row runs the selection above.
__global__ void __launch_bounds__(kSelThreads)
topk_final_kernel(const unsigned long long* __restrict__ comb, const uint2* __restrict__ counts,
                  const uint32_t* __restrict__ hist, int64_t nsp, int nchunk, const int64_t* __restrict__ q_pos,
                  int m, int64_t n_cap, int k, const float* __restrict__ scores, int32_t* __restrict__ topk_idx,
                  float* __restrict__ topk_score) {
  __shared__ FinalShared sh;
  __shared__ uint32_t s_w[kSelThreads / kWave];
  const int64_t r = blockIdx.x;
  final_select(sh, s_w, r, n_visible(q_pos, r, m, n_cap), comb, counts, hist, nsp, nchunk, k, scores, topk_idx,
               topk_score);
}

constexpr int kCandCache = 4096;            // candidate keys kept in LDS during the digit passes
constexpr int kBitmapEntries = 1 << 18;     // rows up to this many entries are ordered through an LDS bitmap
constexpr int kBitmapWords = kBitmapEntries / 32;

struct SelShared {
  uint32_t h256[256];
  uint32_t scan[kSelThreads];
  uint32_t wtot[kSelThreads / kWave];
  int nsel;
  int remaining;
  int done;
  int thr_shift;
  unsigned long long prefix;
  union alignas(16) {
    unsigned long long ckey[kCandCache];      // refine phase
    uint32_t bitmap[kBitmapWords];            // ordering phase
  } u;
};

// Resolve `need` winners among `ncand` candidate keys (all in the threshold bin) digit by digit and
// append their entry indices to sel_list.  Keys are read once into LDS when they fit.
__device__ __forceinline__ void refine_candidates(const unsigned long long* cand, int ncand, int need, int32_t* sel_list,
                                  SelShared& s) {
  const int tid = threadIdx.x;
  const bool cached = ncand <= kCandCache;
  if (cached) {                          // all loads first, then the LDS stores (one round trip)
    constexpr int kPer = kCandCache / kSelThreads;
    unsigned long long v[kPer];
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      v[u] = cand[i < ncand ? i : 0];
    }
#pragma unroll
    for (int u = 0; u < kPer; ++u) {
      const int i = tid + u * kSelThreads;
      if (i < ncand) s.u.ckey[i] = v[u];
    }
  }
  if (tid == 0) { s.remaining = need; s.done = 0; s.prefix = 0ull; s.thr_shift = 0; }
  __syncthreads();
  // the key source is chosen outside the loops (a per-element select would issue the global load too)
  const unsigned long long* src = cand;
  int shift = 53;
  for (int pass = 0; pass < 7; ++pass) {
    const int width = shift >= 8 ? 8 : shift;
    shift -= width;
    for (int i = tid; i < 256; i += kSelThreads) s.h256[i] = 0u;
    __syncthreads();
    const unsigned long long pre = s.prefix;
    if (cached) {
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint64_t key = s.u.ckey[i];
        if ((key >> (shift + width)) == pre) atomicAdd(&s.h256[(key >> shift) & ((1u << width) - 1u)], 1u);
      }
    } else {
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint64_t key = src[i];
        if ((key >> (shift + width)) == pre) atomicAdd(&s.h256[(key >> shift) & ((1u << width) - 1u)], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane j covers digits 255-4j .. 252-4j (top first)
      uint32_t c[4];
      uint32_t lsum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { c[u] = s.h256[255 - 4 * tid - u]; lsum += c[u]; }
      uint32_t incl = lsum;
#pragma unroll
      for (int o = 1; o < kWave; o <<= 1) {
        const uint32_t v = __shfl_up(incl, o, kWave);
        if (tid >= o) incl += v;
      }
      const uint32_t rem = (uint32_t)s.remaining;
      const uint64_t hit = __ballot(incl >= rem);
      const int first = __ffsll((unsigned long long)hit) - 1;
      if (tid == first) {
        uint32_t cum = incl - lsum;
        for (int u = 0; u < 4; ++u) {
          if (cum + c[u] >= rem) {
            const uint32_t d = 255u - 4u * tid - u;
            const uint32_t left = rem - cum;
            s.remaining = (int)left;
            s.prefix = (s.prefix << width) | d;
            if (c[u] == left || shift == 0) { s.done = 1; s.thr_shift = shift; }
            break;
          }
          cum += c[u];
        }
      }
      if (tid == 0 && shift == 0 && !s.done) { s.done = 1; s.thr_shift = 0; }
    }
    __syncthreads();
    if (s.done) break;
  }
  const unsigned long long thr = s.prefix;
  const int ts = s.thr_shift;
  auto take = [&](uint64_t key) {
    if ((key >> ts) >= thr) {
      const int pos = atomicAdd(&s.nsel, 1);
      if (pos < kMaxTopk) sel_list[pos] = (int32_t)(0xFFFFFFFFu - (uint32_t)key);
    }
  };
  if (cached) {
    for (int i = tid; i < ncand; i += kSelThreads) take(s.u.ckey[i]);
  } else {
    for (int i = tid; i < ncand; i += kSelThreads) take(src[i]);
  }
  __syncthreads();
}

// Write the selected entries (unordered, distinct, count n <= 2048) ascending into out[0..k), -1
// padded.  Rows of up to 2^18 entries: set bits in an LDS bitmap and compact it in index order, each
// wave scanning a contiguous range of words 64 at a time.  Longer rows: bitonic sort of the list.
__device__ __forceinline__ void sort_and_write(int32_t* list, int n, int64_t nv, int k, const float* srow,
                               int32_t* out_idx, float* out_score, SelShared& s) {
  const int tid = threadIdx.x;
  const int lane = lane_id();
  const int wave = tid / kWave;
  if (nv <= kBitmapEntries) {
    const int words = (int)((nv + 31) / 32);
    for (int i = tid; i < words; i += kSelThreads) s.u.bitmap[i] = 0u;
    __syncthreads();
    for (int i = tid; i < n; i += kSelThreads) {
      const int32_t e = list[i];
      if (e >= 0 && (int64_t)e < nv) atomicOr(&s.u.bitmap[e >> 5], 1u << (e & 31));
    }
    __syncthreads();
    // Thread t owns words [32t, 32t + 32) (entries 1024t ..): its bits go to registers, one block-wide
    // exclusive scan of the per-thread counts gives its output offset, then it writes its entries
    // in index order.
    constexpr int kWordsPerThread = kBitmapWords / kSelThreads;            // 32
    static_assert(kWordsPerThread % 4 == 0, "whole uint4 reads per thread");
    uint32_t bits[kWordsPerThread];
    const int w0 = tid * kWordsPerThread;
#pragma unroll
    for (int q = 0; q < kWordsPerThread / 4; ++q) {
      const uint4 x = *reinterpret_cast<const uint4*>(&s.u.bitmap[w0 + 4 * q]);
      bits[4 * q + 0] = w0 + 4 * q + 0 < words ? x.x : 0u;
      bits[4 * q + 1] = w0 + 4 * q + 1 < words ? x.y : 0u;
      bits[4 * q + 2] = w0 + 4 * q + 2 < words ? x.z : 0u;
      bits[4 * q + 3] = w0 + 4 * q + 3 < words ? x.w : 0u;
    }
    uint32_t cnt = 0;
#pragma unroll
    for (int q = 0; q < kWordsPerThread; ++q) cnt += (uint32_t)__popc(bits[q]);
    uint32_t incl = cnt;
#pragma unroll
    for (int o = 1; o < kWave; o <<= 1) {
      const uint32_t v = __shfl_up(incl, o, kWave);
      if (lane >= o) incl += v;
    }
    if (lane == kWave - 1) s.wtot[wave] = incl;
    __syncthreads();
    uint32_t pos = incl - cnt;
    for (int v = 0; v < wave; ++v) pos += s.wtot[v];
#pragma unroll
    for (int q = 0; q < kWordsPerThread; ++q) {
      uint32_t b = bits[q];
      while (b) {
        const int e = (w0 + q) * 32 + __ffs(b) - 1;
        b &= b - 1;
        out_idx[pos] = e;
        if (out_score) out_score[pos] = srow[e];
        ++pos;
      }
    }
  } else {
    int P = 2;
    while (P < n) P <<= 1;
    for (int i = tid; i < P; i += kSelThreads) if (i >= n) list[i] = INT_MAX;
    __syncthreads();
    constexpr int kPairs = kMaxTopk / 2 / kSelThreads;         // pairs per thread per phase (<= 4)
    for (int kk = 2; kk <= P; kk <<= 1) {
      for (int j = kk >> 1; j > 0; j >>= 1) {
        int32_t x[kPairs], y[kPairs];
        int ii[kPairs];
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {                     // all reads of the phase first
          const int p = tid + u * kSelThreads;
          ii[u] = ((p & ~(j - 1)) << 1) | (p & (j - 1));
          const bool act = p < (P >> 1);
          x[u] = act ? list[ii[u]] : 0;
          y[u] = act ? list[ii[u] + j] : 0;
        }
#pragma unroll
        for (int u = 0; u < kPairs; ++u) {
          const int p = tid + u * kSelThreads;
          if (p < (P >> 1)) {
            const bool up = (ii[u] & kk) == 0;
            if ((x[u] > y[u]) == up) { list[ii[u]] = y[u]; list[ii[u] + j] = x[u]; }
          }
        }
        __syncthreads();
      }
    }
    for (int i = tid; i < n; i += kSelThreads) {
      out_idx[i] = list[i];
      if (out_score) out_score[i] = srow[list[i]];
    }
  }
  for (int i = n + tid; i < k; i += kSelThreads) {
    out_idx[i] = -1;
    if (out_score) out_score[i] = -INFINITY;
  }
}

// Prefill: one workgroup per row does histogram, filter, refine, sort.
__global__ void __launch_bounds__(kSelThreads)
topk_rowwise_kernel(const float* __restrict__ scores, unsigned long long* __restrict__ cand, int64_t nsp,
                    const int64_t* __restrict__ q_pos, int m, int64_t n_cap, int k,
                    int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelShared s;
  __shared__ int32_t list[kMaxTopk];
  __shared__ __align__(16) uint32_t h[kBins];
  __shared__ int sT, sAbove, sCand;
  const int tid = threadIdx.x;
  const int64_t r = blockIdx.x;
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const float* srow = scores + r * nsp;
  if (nv <= k) {
    for (int64_t i = tid; i < k; i += kSelThreads) {
      topk_idx[r * k + i] = i < nv ? (int32_t)i : -1;
      if (topk_score) topk_score[r * k + i] = i < nv ? srow[i] : -INFINITY;
    }
    return;
  }
  for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0u;
  if (tid == 0) { s.nsel = 0; sCand = 0; sT = kBins - 1; sAbove = 0; }
  __syncthreads();
  for (int64_t e = tid; e < nv; e += kSelThreads) atomicAdd(&h[float_key(srow[e]) >> kBinShift], 1u);
  __syncthreads();
  find_threshold(h, k, &sT, &sAbove, s.scan);
  const int T = sT;
  unsigned long long* crow = cand + r * nsp;
  for (int64_t e = tid; e < nv; e += kSelThreads) {
    const uint32_t key = float_key(srow[e]);
    const int bin = (int)(key >> kBinShift);
    if (bin > T) list[atomicAdd(&s.nsel, 1)] = (int32_t)e;
    else if (bin == T) crow[atomicAdd(&sCand, 1)] = cand_key(key, (int32_t)e);
  }
  __syncthreads();
  const int nsel = s.nsel;
  refine_candidates(crow, sCand, k - nsel, list, s);
  const int n = s.nsel < k ? s.nsel : k;
  sort_and_write(list, n, nv, k, srow, topk_idx + r * k, topk_score ? topk_score + r * k : nullptr, s);
}

// Entries per decode scoring workgroup: about two workgroups per CU over the whole call.
int64_t decode_chunk(int64_t n_cap, int R) {
  int64_t c = (n_cap * R + 511) / 512;
  c = (c + 255) & ~(int64_t)255;
  if (c < 256) c = 256;
  if (c > 65536) c = 65536;
  return c;
}

template <bool FP8, int KS, int HBI, int QW>
void launch_score(const IndexArgs& a, const Ws& w, hipStream_t st) {
  if constexpr (QW == 1) {
    const int64_t chunk = decode_chunk(a.n_cap, a.B * a.Tq);
    dim3 grid((unsigned)((a.n_cap + chunk - 1) / chunk), (unsigned)(a.B * a.Tq));
    LCS_LAUNCH("index_score_kernel", (index_score_decode_kernel<FP8, KS, HBI>), grid, dim3(256), 0, st,
               a.q_idx, a.w_idx, a.ik, a.ik_scale, a.ik_ld, a.q_pos, a.n_cap, a.Tq, a.H_I, a.dI, a.m, chunk,
               w.scores, w.hist, w.nsp);
    return;
  }
  constexpr int QTILE = QW == 1 ? 1 : 16;
  const int tiles = (a.Tq + QTILE - 1) / QTILE;
  dim3 grid((unsigned)((a.n_cap + kScoreChunk - 1) / kScoreChunk), (unsigned)(a.B * tiles));
  LCS_LAUNCH("index_score_kernel", (index_score_kernel<FP8, KS, HBI, QW>), grid, dim3(256), 0, st,
             a.q_idx, a.w_idx, a.ik, a.ik_scale, a.ik_ld, a.q_pos, a.n_cap, a.Tq, a.H_I, a.dI, a.m,
             w.scores, w.hist, w.nsp);
}

template <bool FP8, int KS, int QW>
void dispatch_hbi(const IndexArgs& a, const Ws& w, hipStream_t st) {
  if (a.H_I <= 16) launch_score<FP8, KS, 1, QW>(a, w, st);
  else if (a.H_I <= 32) launch_score<FP8, KS, 2, QW>(a, w, st);
  else launch_score<FP8, KS, 4, QW>(a, w, st);
}

template <int QW>
void dispatch_score(const IndexArgs& a, const Ws& w, hipStream_t st) {
  if (a.ik_fp8) dispatch_hbi<true, 1, QW>(a, w, st);
  else if (a.dI == 64) dispatch_hbi<false, 2, QW>(a, w, st);
  else dispatch_hbi<false, 4, QW>(a, w, st);
}

}  // namespace

size_t index_topk_workspace(int B, int Tq, int64_t n_cap, int k) {
  (void)k;
  const int64_t R = (int64_t)B * Tq;
  const int64_t nsp = (n_cap + 63) & ~(int64_t)63;
  return al256((size_t)R * nsp * 4) + al256((size_t)R * kHistRow * 4) + al256((size_t)R * nsp * 8) +
         al256((size_t)R * n_chunks(n_cap) * 8);
}

int launch_index_topk(const IndexArgs& a, hipStream_t st) {
  const int R = a.B * a.Tq;
  Ws w = carve(a.ws, R, a.n_cap);
  // Few rows: spread every row over many workgroups (decode).  Many rows, or rows longer than the
  // decode selection stages: row-per-workgroup.
  const bool decode = R < 64 && w.nchunk <= kMaxDecodeChunks;
  if (decode) {
    const int64_t n = (int64_t)R * kHistRow;
    LCS_LAUNCH("topk_clear_kernel", clear_u32_kernel, dim3((unsigned)((n + 255) / 256 < 1024 ? (n + 255) / 256 : 1024)),
               dim3(256), 0, st, w.hist, n);
    dispatch_score<1>(a, w, st);
    dim3 gf((unsigned)w.nchunk, (unsigned)R);
    LCS_LAUNCH("topk_filter_kernel", topk_filter_kernel, gf, dim3(kSelThreads), 0, st, w.scores, w.hist, w.comb,
               w.counts, w.nsp, w.nchunk, a.q_pos, a.m, a.n_cap, a.k);
    LCS_LAUNCH("topk_final_kernel", topk_final_kernel, dim3((unsigned)R), dim3(kSelThreads), 0, st, w.comb,
               w.counts, w.hist, w.nsp, w.nchunk, a.q_pos, a.m, a.n_cap, a.k, w.scores, a.topk_idx, a.topk_score);
  } else {
    dispatch_score<4>(a, w, st);
    LCS_LAUNCH("topk_rowwise_kernel", topk_rowwise_kernel, dim3((unsigned)R), dim3(kSelThreads), 0, st, w.scores,
               w.comb, w.nsp, a.q_pos, a.m, a.n_cap, a.k, a.topk_idx, a.topk_score);
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
