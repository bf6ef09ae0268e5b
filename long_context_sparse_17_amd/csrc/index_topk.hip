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
#include "decode_append.h"
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
constexpr int kMaxIndexHeads = 64;         // indexer heads (the entry point rejects more)

inline size_t al256(size_t x) { return (x + 255) & ~(size_t)255; }

// Decode selection keeps per-row histograms in a fixed area at the start of the workspace, for up
// to kDecodeRows rows.  The area is zero between calls: the caller zero-fills the workspace once, the
// scorer and filter add into the rows a call uses, and the final kernel clears them again, so no call
// needs a clearing launch of its own.
constexpr int kDecodeRows = 64;
constexpr int kMaxDecodeChunks = 2048;       // decode selection: rows up to 8M entries

struct Ws {
  uint32_t* hist;                 // [kDecodeRows, kHistRow]: histograms of the top score-key bits, then of the next 11
  float* scores;                  // [RS, nsp] (RS: every row at decode, one batch of queries in prefill)
  unsigned long long* comb;       // [RS, nsp]: kept entries per chunk (decode) / candidates (prefill)
  uint2* counts;                  // [R, nchunk]: per decode chunk (kept, above the threshold bin)
  uint8_t* qc;                    // [R, HP, 128]: E4M3FN query codes (fp8 prefill)
  float* qw;                      // [R, HP]: head weights times the query row scales (fp8 prefill)
  int32_t* qnv;                   // [R]: visible entries per row (fp8 prefill)
  uint8_t* linc;                  // [B * ceil(Tq / 4), 16, 128]: linear-term parts (fp8 prefill)
  uint32_t* lins;                 // [B * ceil(Tq / 4), 16, 4]: their scale exponents (E8M0)
  int64_t nsp;
  int nchunk;
};

inline int64_t n_chunks(int64_t n_cap) { return (n_cap + kFilterChunk - 1) / kFilterChunk; }

// Rows of many queries (prefill) are scored and selected in batches of queries: each batch takes
// query positions [t0, t0 + tb) of every batch row, so the score and candidate buffers hold B * tb
// rows whatever Tq is.  tb is a multiple of 16 (the bf16 scorer's query tile, and a multiple of the
// fp8 scorer's 4-query stage) unless one batch covers all of Tq.  768 rows are one round of the
// selection kernel (3 workgroups per CU on 256 CUs): a batch that leaves a partial second round
// costs more than the extra launches.  Calls whose buffers for all rows (12 bytes per row and
// entry) stay within kPfOneBatchBytes run as one batch: there the launches of more batches cost more
// than the buffers save.
constexpr int kPfBatchRows = 768;
constexpr int64_t kPfOneBatchBytes = (int64_t)64 << 20;
inline int prefill_batch(int B, int Tq, int64_t n_cap) {
  const int want = kPfBatchRows / B;
  const int64_t nsp = (n_cap + 63) & ~(int64_t)63;
  if (Tq <= want || Tq <= 16 || (int64_t)B * Tq * nsp * 12 <= kPfOneBatchBytes) return Tq;
  const int tb = want / 16 * 16;
  return tb < 16 ? 16 : tb;
}
inline bool decode_rows(int B, int Tq, int64_t n_cap) {
  return (int64_t)B * Tq < kDecodeRows && n_chunks(n_cap) <= kMaxDecodeChunks;
}
// rows of the score and candidate buffers: every row at decode, one batch of queries otherwise
inline int64_t buffer_rows(int B, int Tq, int64_t n_cap) {
  return decode_rows(B, Tq, n_cap) ? (int64_t)B * Tq : (int64_t)B * prefill_batch(B, Tq, n_cap);
}

inline int64_t n_groups4(int B, int Tq) { return (int64_t)B * ((Tq + 3) / 4); }

Ws carve(void* ws, int B, int Tq, int64_t n_cap) {
  const int R = B * Tq;
  const int64_t RS = buffer_rows(B, Tq, n_cap);
  Ws w;
  w.nsp = (n_cap + 63) & ~(int64_t)63;
  w.nchunk = (int)n_chunks(n_cap);
  char* p = static_cast<char*>(ws);
  w.hist = reinterpret_cast<uint32_t*>(p);
  p += al256((size_t)kDecodeRows * kHistRow * 4);
  w.scores = reinterpret_cast<float*>(p);
  p += al256((size_t)RS * w.nsp * 4);
  w.comb = reinterpret_cast<unsigned long long*>(p);
  p += al256((size_t)RS * w.nsp * 8);
  w.counts = reinterpret_cast<uint2*>(p);
  p += al256((size_t)R * w.nchunk * 8);
  w.qc = reinterpret_cast<uint8_t*>(p);
  p += al256((size_t)R * kMaxIndexHeads * 128);
  w.qw = reinterpret_cast<float*>(p);
  p += al256((size_t)R * kMaxIndexHeads * 4);
  w.qnv = reinterpret_cast<int32_t*>(p);
  p += al256((size_t)R * 4);
  w.linc = reinterpret_cast<uint8_t*>(p);
  p += al256((size_t)n_groups4(B, Tq) * 2048);
  w.lins = reinterpret_cast<uint32_t*>(p);
  return w;
}

__device__ __forceinline__ int64_t n_visible(const int64_t* q_pos, int64_t r, int m, int64_t n_cap) {
  int64_t t = q_pos[r];
  int64_t n = t >= 0 ? t / m : 0;
  return n < n_cap ? n : n_cap;
}

// ------------------------------------------------------------------------------------ scoring
// 32 dims of one head row -- the 16 at qseg0, then the 16 at qseg1 (the row's 4 lane groups together
// hold all 128 dims) -- quantised to E4M3FN with the row's scale absmax / 448 (RNE, correctly rounded
// division: the decision rule the selection depends on), packed in that order as an MFMA A fragment.
// Returns the row scale (1 for an all-zero row).  hv == false: zero codes (padding heads).  The
// matrix cores only need A and B to share one assignment of dims to (lane group, register, byte).
// The two 16-dim segments of a row (unconditional loads; a padding head's values are dropped later).
__device__ __forceinline__ void load_row_segments(const uint16_t* qseg0, const uint16_t* qseg1, uint4 (&raw)[4]) {
#pragma unroll
  for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const uint4*>((u < 2 ? qseg0 : qseg1) + 8 * (u & 1));
}
__device__ __forceinline__ float quant_loaded_e4m3(const uint4 (&loaded)[4], bool hv, intx8& codes) {
  uint4 raw[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) raw[u] = hv ? loaded[u] : make_uint4(0, 0, 0, 0);
  float amax = 0.f;
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const uint32_t wd[4] = {raw[u].x, raw[u].y, raw[u].z, raw[u].w};
#pragma unroll
    for (int j = 0; j < 4; ++j) amax = fmaxf(amax, fmaxf(fabsf(bf2f_lo(wd[j])), fabsf(bf2f_hi(wd[j]))));
  }
  amax = max_rows4(amax);
  const float sc = amax > 0.f ? __fdiv_rn(amax, 448.0f) : 1.0f;
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
  return sc;
}
__device__ __forceinline__ float quant_row_e4m3(const uint16_t* qseg0, const uint16_t* qseg1, bool hv, intx8& codes) {
  uint4 raw[4];
  load_row_segments(qseg0, qseg1, raw);                 // callers pass a valid row for padding heads
  return quant_loaded_e4m3(raw, hv, codes);
}

// bf16 keys, many query rows (prefill with bf16 indexer keys): 16 queries per workgroup, 4 per wave;
// every wave scores the workgroup's whole chunk (`chunk` entries, a multiple of 64) for its 4 queries
// (entries re-read from L1/L2).
template <int KS, int HBI>
__global__ void __launch_bounds__(256)
index_score_kernel(const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w_idx,
                   const uint16_t* __restrict__ ik, int64_t ik_ld, const int64_t* __restrict__ q_pos,
                   int64_t n_cap, int Tq, int t0, int tcur, int tb, int H_I, int dI, int m,
                   float* __restrict__ scores, int64_t nsp, int chunk) {
  constexpr int QW = 4, QTILE = 16;
  const int lane = lane_id();
  const int wave = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  // query positions [t0, t0 + tcur) of every batch row; scores to buffer rows b * tb + (t - t0)
  const int tiles_per_b = (tcur + QTILE - 1) / QTILE;
  const int b = blockIdx.y / tiles_per_b;
  const int tq0 = t0 + (blockIdx.y % tiles_per_b) * QTILE;
  const int tq_end = t0 + tcur < Tq ? t0 + tcur : Tq;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;

  // entry limit of this workgroup = max n_vis over its queries
  int64_t nv_max = 0;
  for (int i = 0; i < QTILE; ++i) {
    const int tq = tq0 + i;
    if (tq < tq_end) {
      const int64_t nv = n_visible(q_pos, (int64_t)b * Tq + tq, m, n_cap);
      nv_max = nv > nv_max ? nv : nv_max;
    }
  }
  if (c0 >= nv_max) return;                    // uniform across the workgroup

  uint4 afr[QW][HBI][KS];
  float wq[QW][HBI][4];
  int64_t nvis[QW];
  int64_t rowq[QW];                            // buffer row of each query
#pragma unroll
  for (int qw = 0; qw < QW; ++qw) {
    const int tq = tq0 + wave * QW + qw;
    const bool qvalid = tq < tq_end;
    const int64_t r = (int64_t)b * Tq + (qvalid ? tq : t0);
    rowq[qw] = (int64_t)b * tb + ((qvalid ? tq : t0) - t0);
    nvis[qw] = qvalid ? n_visible(q_pos, r, m, n_cap) : 0;
#pragma unroll
    for (int hb = 0; hb < HBI; ++hb) {
      const int head = hb * 16 + c16;
      const bool hv = qvalid && head < H_I;
      const uint16_t* qrow = q_idx + (r * H_I + (hv ? head : 0)) * dI;
      const float wh = hv ? bf2f(w_idx[r * H_I + head]) : 0.f;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        afr[qw][hb][ks] = hv ? *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
      // the D fragment of this lane holds heads 16hb + 4g + i: fetch their weights
#pragma unroll
      for (int i = 0; i < 4; ++i) wq[qw][hb][i] = __shfl(wh, 4 * g + i, kWave);
    }
  }

  int64_t e_hi = c0 + chunk;
  if (e_hi > nv_max) e_hi = nv_max;
  const uint16_t* ik16 = ik + (int64_t)b * ik_ld * dI;
  for (int64_t e0 = c0; e0 < e_hi; e0 += 64) {
    uint4 bfr[4][KS];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int64_t e = e0 + 16 * u + c16;
#pragma unroll
      for (int ks = 0; ks < KS; ++ks)
        bfr[u][ks] = e < e_hi ? *reinterpret_cast<const uint4*>(ik16 + e * dI + 32 * ks + 8 * g) : make_uint4(0, 0, 0, 0);
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
          for (int ks = 0; ks < KS; ++ks) acc = mfma_bf16(afr[qw][hb][ks], bfr[u][ks], acc);
#pragma unroll
          for (int i = 0; i < 4; ++i) part += wq[qw][hb][i] * fmaxf(acc[i], 0.f);
        }
        part = sum_rows4(part);
        const int64_t e = e0 + 16 * u + c16;
        if (g == 0 && e < nvis[qw]) scores[rowq[qw] * nsp + e] = part + 0.0f;
      }
    }
  }
}

// fp8 keys, many query rows (chunked prefill).  The head sum is evaluated through
//     sum_h w'_h relu(a_h) = 1/2 sum_h w'_h |a_h|  +  1/2 sum_h w'_h a_h          (w'_h = w_h * s_h)
// where a_h = q^_h . k is the code dot product of head h: the first half costs one fused multiply-add
// per head and entry (|a| is a free source modifier), the second is linear in the query,
// (sum_h w'_h q^_h / 2) . k = u . k, and runs on the matrix cores.  u (128 values per query) is
// carried as 4 E4M3FN parts with one power-of-two (E8M0) scale each, every part encoding the previous
// parts' exact residual, so |u - sum of parts| <= 2^-19 max|u| elementwise.  Two
// kernels:
//   index_qprep_kernel: every query head row quantised once (codes [R][HP][128] in fragment order,
//     half weights w'_h / 2 [R][HP], HP = heads padded to 16 with zero codes and weights), each
//     row's visible entry count (int32), and the parts of u as the rows 4j + p of one MFMA A fragment
//     per 4 consecutive queries (codes [G][16][128], scale exponents [G][16][4] (all four equal),
//     G = (b, t / 4)).
//   index_score_prefill_kernel: one workgroup of 8 waves per chunk of 1024 entries (and a range of
//     queries).  Each wave keeps the B fragments of its 128 entries (8 blocks of 16) in registers for
//     the whole launch and streams the queries: stages of 4 queries' codes and weights go through LDS
//     (double-buffered, one barrier per stage); per stage 8 MFMAs give the 4 queries' u . k (lane
//     group j holds query j's parts), per query each head block's A fragment feeds 8 MFMAs back to
//     back, |a| * w'/2 accumulates per entry block onto query j's linear term (lane group j only), and
//     a reduce-scatter over the 4 lane groups (v_permlane16/32_swap) leaves lane (g, c) with entry
//     blocks g and 4 + g, so each query's 128 scores leave in two 256-byte row stores.
constexpr int kPfWaves = 8;
constexpr int kPfEB = 8;                                // 16-entry blocks per wave
constexpr int kPfChunk = kPfWaves * kPfEB * 16;         // entries per workgroup
constexpr int kPfQC = 4;                                // queries per LDS stage
constexpr int kPfRow = 144;                             // LDS bytes per head row: 128 codes + 16 (conflict-free reads)

constexpr int kLinParts = 4;                            // E4M3FN parts of the linear-term vector u

// E4M3FN code -> value, exact: bias 7, 3 mantissa bits, subnormal quantum 2^-9 (no NaN codes occur).
__device__ __forceinline__ double e4m3_value(uint32_t c) {
  const int e = (int)((c >> 3) & 15u), mt = (int)(c & 7u);
  const double v = e ? ldexp(8.0 + mt, e - 10) : ldexp((double)mt, -9);
  return (c & 0x80u) ? -v : v;
}

template <int HBI>
__global__ void __launch_bounds__(256)
index_qprep_kernel(const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w_idx, int H_I,
                   const int64_t* __restrict__ q_pos, int64_t n_cap, int m, int Tq, uint8_t* __restrict__ qc,
                   float* __restrict__ qwf, int32_t* __restrict__ qnv, uint8_t* __restrict__ linc,
                   uint32_t* __restrict__ lins) {
  constexpr int HP = 16 * HBI;
  __shared__ uint32_t s_codes[HP][33];                 // a head row's 128 codes as 32 words (+1: no conflicts)
  __shared__ float s_w[HP];
  const int lane = lane_id(), wave = threadIdx.x / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t r = blockIdx.x;
  if (wave < HBI) {
    const int head = 16 * wave + c16;
    const bool hv = head < H_I;
    intx8 codes;
    const uint16_t* qrow = q_idx + (r * H_I + (hv ? head : 0)) * 128;
    const float sc = quant_row_e4m3(qrow + 32 * g, qrow + 32 * g + 16, hv, codes);
    uint4* dst = reinterpret_cast<uint4*>(qc + (r * HP + head) * 128 + 32 * g);
    dst[0] = make_uint4((uint32_t)codes[0], (uint32_t)codes[1], (uint32_t)codes[2], (uint32_t)codes[3]);
    dst[1] = make_uint4((uint32_t)codes[4], (uint32_t)codes[5], (uint32_t)codes[6], (uint32_t)codes[7]);
    const float wh = hv ? bf2f(w_idx[r * H_I + head]) * sc * 0.5f : 0.f;
    if (g == 0) {
      qwf[r * HP + head] = wh;
      s_w[head] = wh;
    }
#pragma unroll
    for (int i = 0; i < 8; ++i) s_codes[head][8 * g + i] = (uint32_t)codes[i];
  }
  if (threadIdx.x == 0) qnv[r] = (int32_t)n_visible(q_pos, r, m, n_cap);
  __syncthreads();
  // u_d = sum_h (w'_h / 2) * value(code_hd) in fp64 (exact products, 64 terms), then split into parts:
  // part p = RNE_e4m3(res / 2^e_p) with e_p the smallest exponent putting the row's largest |res|
  // within 448, res -= 2^e_p * part (exact).  One exponent per part and query: the matrix cores'
  // 32-value scale blocks follow their own k order, so the same exponent goes to all four.
  // Dims d = threadIdx.x < 128 (waves 0, 1); every thread takes part in the barriers.
  __shared__ double s_mx[2];
  const int d = threadIdx.x;
  double res = 0.0;
  if (d < 128)
    for (int h = 0; h < HP; ++h)
      res += (double)s_w[h] * e4m3_value((s_codes[h][d >> 2] >> (8 * (d & 3))) & 0xFFu);
  const int64_t b = r / Tq;
  const int tq = (int)(r % Tq), j = tq & 3;
  const int64_t G = b * ((Tq + 3) / 4) + tq / 4;
  uint8_t* crow = linc + G * 2048;
  uint32_t* srow = lins + G * 64;
#pragma unroll 1
  for (int p = 0; p < kLinParts; ++p) {
    double mx = d < 128 ? fabs(res) : 0.0;
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) mx = fmax(mx, __shfl_xor(mx, o, kWave));
    if (lane == 0 && wave < 2) s_mx[wave] = mx;
    __syncthreads();
    mx = fmax(s_mx[0], s_mx[1]);
    __syncthreads();                                   // s_mx is rewritten by the next part
    int e = 0;
    if (mx > 0.0) {
      int k;
      const double f = frexp(mx / 448.0, &k);          // mx / 448 = f 2^k, f in [0.5, 1)
      e = f == 0.5 ? k - 1 : k;
      e = e < -127 ? -127 : (e > 127 ? 127 : e);
    }
    if (d < 128) {
      const uint32_t c = f2e4m3((float)ldexp(res, -e));
      res -= ldexp(e4m3_value(c), e);
      crow[(4 * j + p) * 128 + d] = (uint8_t)c;
    }
    if (d < 4) srow[(4 * j + p) * 4 + d] = (uint32_t)(e + 127);
  }
  // the last query of a partial group clears the rows of the missing ones
  if (tq == Tq - 1 && d < 128) {
    for (int jj = j + 1; jj < 4; ++jj)
      for (int p = 0; p < kLinParts; ++p) {
        crow[(4 * jj + p) * 128 + d] = 0;
        if (d < 4) srow[(4 * jj + p) * 4 + d] = 127u;
      }
  }
}

template <int HBI>
__global__ void __launch_bounds__(kPfWaves * kWave)
index_score_prefill_kernel(const uint8_t* __restrict__ qc, const float* __restrict__ qwf,
                           const int32_t* __restrict__ qnv, const uint8_t* __restrict__ linc,
                           const uint32_t* __restrict__ lins, const uint8_t* __restrict__ ik,
                           const float* __restrict__ ik_scale, int64_t ik_ld, int64_t n_cap, int Tq, int t0,
                           int tcur, int tb, int qsplit, int qper, float* __restrict__ scores, int64_t nsp) {
  constexpr int HP = 16 * HBI;
  constexpr int kCodeBytes = HP * kPfRow;
  constexpr int kSlot = kCodeBytes + HP * 4 + 16;      // one query in LDS: codes, folded weights, n_vis
  constexpr int kThreads = kPfWaves * kWave;
  constexpr int kLd = kPfQC * HP * 8 / kThreads;       // 16-byte code pieces per thread per stage (= HBI)
  static_assert(kPfQC * HP * 8 == kLd * kThreads, "stage pieces must divide evenly");
  static_assert(kPfQC * (HP + 1) <= kThreads, "one weight or count per thread");
  static_assert(kPfQC == 4 && kLinParts == 4, "a stage's linear-term fragment holds 4 queries x 4 parts");
  __shared__ __align__(16) uint8_t sq[2][kPfQC][kSlot];

  const int tid = threadIdx.x, lane = lane_id(), wave = tid / kWave;
  const int g = lane >> 4, c16 = lane & 15;
  // this launch scores query positions [t0, t0 + tcur) of every batch row; their scores go to buffer
  // rows b * tb + (t - t0)
  const int b = blockIdx.y / qsplit;
  const int q_lo = t0 + (blockIdx.y % qsplit) * qper;
  const int q_end = t0 + tcur < Tq ? t0 + tcur : Tq;
  const int q_hi = q_lo + qper < q_end ? q_lo + qper : q_end;
  if (q_lo >= q_hi) return;                            // uniform
  const int64_t c0 = (int64_t)blockIdx.x * kPfChunk;
  const int64_t ew = c0 + wave * (kPfEB * 16);         // first entry of this wave

  // ---- this wave's keys: B fragments (entry 16 eb + c16, dims [32g, 32g + 32)) and two scales ----
  intx8 bfr[kPfEB];
  const uint8_t* ikb = ik + (int64_t)b * ik_ld * 128;
#pragma unroll
  for (int eb = 0; eb < kPfEB; ++eb) {
    const int64_t e = ew + 16 * eb + c16;
    uint4 x0 = make_uint4(0, 0, 0, 0), x1 = x0;
    if (e < n_cap) {
      const uint4* p = reinterpret_cast<const uint4*>(ikb + e * 128 + 32 * g);
      x0 = p[0];
      x1 = p[1];
    }
    bfr[eb] = intx8{(int)x0.x, (int)x0.y, (int)x0.z, (int)x0.w, (int)x1.x, (int)x1.y, (int)x1.z, (int)x1.w};
  }
  const int64_t e_lo = ew + 16 * g + c16;              // entries this lane stores: e_lo, e_lo + 64
  const float* ksb = ik_scale + (int64_t)b * ik_ld;
  const float ks0 = e_lo < n_cap ? ksb[e_lo] : 0.f;
  const float ks1 = e_lo + 64 < n_cap ? ksb[e_lo + 64] : 0.f;

  // ---- query stages: codes, weights and n_vis of kPfQC queries, global -> registers -> LDS.  Slots
  // past the range load the range's last query (never scored), so every load is unconditional. ----
  // staging registers as one native vector: an array of uint4 here is not promoted to registers
  // (it would live in scratch and the prefetch would wait for its loads at once)
  typedef uint32_t u32x16 __attribute__((ext_vector_type(16)));
  static_assert(kLd <= 4, "staging vector holds 4 pieces");
  u32x16 stg;
  uint32_t stw = 0u;
  const int64_t row0 = (int64_t)b * Tq;
  const int64_t G0 = (int64_t)b * ((Tq + 3) / 4) + q_lo / 4;  // linear-term fragment of stage 0
  uint4 lx0, lx1;                                      // next stage's fragment: this lane's 32 codes ...
  uint32_t lxs;                                        // ... and their scale exponent
#define LCS_PF_FETCH(S)                                                                           \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < kLd; ++i) {                                             \
      const int c = tid + i * kThreads; /* piece index in [kPfQC][HP][8] */                       \
      const int j = c / (HP * 8), head = (c / 8) % HP, piece = c % 8;                             \
      int tq = q_lo + (S) * kPfQC + j;                                                            \
      tq = tq < q_hi ? tq : q_hi - 1;                                                             \
      const uint4 t = *reinterpret_cast<const uint4*>(qc + ((row0 + tq) * HP + head) * 128 + 16 * piece); \
      stg[4 * i] = t.x; stg[4 * i + 1] = t.y; stg[4 * i + 2] = t.z; stg[4 * i + 3] = t.w;        \
    }                                                                                             \
    {                                                                                             \
      const uint4* lp = reinterpret_cast<const uint4*>(linc + (G0 + (S)) * 2048 + c16 * 128 + 32 * g); \
      lx0 = lp[0];                                                                                \
      lx1 = lp[1];                                                                                \
      lxs = lins[(G0 + (S)) * 64 + c16 * 4 + g];                                                  \
    }                                                                                             \
    if (tid < kPfQC * HP) {                                                                       \
      int tq = q_lo + (S) * kPfQC + tid / HP;                                                     \
      tq = tq < q_hi ? tq : q_hi - 1;                                                             \
      stw = __float_as_uint(qwf[(row0 + tq) * HP + tid % HP]);                                    \
    } else if (tid < kPfQC * (HP + 1)) {                                                          \
      int tq = q_lo + (S) * kPfQC + (tid - kPfQC * HP);                                           \
      tq = tq < q_hi ? tq : q_hi - 1;                                                             \
      stw = (uint32_t)qnv[row0 + tq];                                                             \
    }                                                                                             \
  } while (0)
#define LCS_PF_COMMIT(BUF)                                                                        \
  do {                                                                                            \
    _Pragma("unroll") for (int i = 0; i < kLd; ++i) {                                             \
      const int c = tid + i * kThreads;                                                           \
      const int j = c / (HP * 8), head = (c / 8) % HP, piece = c % 8;                             \
      *reinterpret_cast<uint4*>(&sq[BUF][j][head * kPfRow + 16 * piece]) =                       \
          make_uint4(stg[4 * i], stg[4 * i + 1], stg[4 * i + 2], stg[4 * i + 3]);                \
    }                                                                                             \
    if (tid < kPfQC * HP)                                                                         \
      *reinterpret_cast<uint32_t*>(&sq[BUF][tid / HP][kCodeBytes + 4 * (tid % HP)]) = stw;        \
    else if (tid < kPfQC * (HP + 1))                                                              \
      *reinterpret_cast<uint32_t*>(&sq[BUF][tid - kPfQC * HP][kCodeBytes + 4 * HP]) = stw;        \
  } while (0)

  const int nst = (q_hi - q_lo + kPfQC - 1) / kPfQC;
  LCS_PF_FETCH(0);
  LCS_PF_COMMIT(0);
  __syncthreads();
  for (int s = 0; s < nst; ++s) {
    const intx8 la = intx8{(int)lx0.x, (int)lx0.y, (int)lx0.z, (int)lx0.w, (int)lx1.x, (int)lx1.y, (int)lx1.z, (int)lx1.w};
    const int lsc = (int)lxs;
    if (s + 1 < nst) LCS_PF_FETCH(s + 1);              // in flight while this stage is scored
    const uint8_t* qb = &sq[s & 1][0][0];
    int nvq[kPfQC];
    int nv_hi = 0;
#pragma unroll
    for (int j = 0; j < kPfQC; ++j) {
      const int v = __builtin_amdgcn_readfirstlane(*reinterpret_cast<const int32_t*>(qb + j * kSlot + kCodeBytes + 4 * HP));
      nvq[j] = q_lo + s * kPfQC + j < q_hi ? v : 0;
      nv_hi = nvq[j] > nv_hi ? nvq[j] : nv_hi;
    }
    if (ew < nv_hi) {                                  // wave-uniform: some entry of this wave visible
      // u . k of the stage's 4 queries: lane group j holds query j's 4 parts; their sum is its term
      float lin[kPfEB];
#pragma unroll
      for (int eb = 0; eb < kPfEB; ++eb) {
        const floatx4 t = mfma_fp8_scale_a(la, bfr[eb], lsc);
        lin[eb] = (t[0] + t[1]) + (t[2] + t[3]);
      }
      // Straight-line software pipeline over the stage's steps (query j, head block hb): the MFMAs
      // of step t are issued next to the |a| * w' accumulation of step t - 1, whose results are
      // long complete, so the in-order issue never waits on a fresh MFMA result.  Invisible
      // queries of a partly visible stage are computed and not stored.
      constexpr int NSTEP = kPfQC * HBI;
      floatx4 acc[2][kPfEB];
      intx8 av[2];
      float4 wv[3];                                    // step t's weights are read at t - 1 and used at t + 1
      float part[kPfEB];
      float res0[kPfQC], res1[kPfQC];
      auto read_step = [&](int t) {                    // A fragment and head weights of step t (LDS)
        const int j = t / HBI, hb = t % HBI;
        const uint8_t* qs = qb + j * kSlot;
        const uint4* ap = reinterpret_cast<const uint4*>(qs + (16 * hb + c16) * kPfRow + 32 * g);
        const uint4 a0 = ap[0], a1 = ap[1];
        av[t & 1] = intx8{(int)a0.x, (int)a0.y, (int)a0.z, (int)a0.w, (int)a1.x, (int)a1.y, (int)a1.z, (int)a1.w};
        wv[t % 3] = *reinterpret_cast<const float4*>(qs + kCodeBytes + 4 * (16 * hb + 4 * g));
      };
      read_step(0);
#pragma unroll
      for (int t = 0; t <= NSTEP; ++t) {
        if (t + 1 < NSTEP) read_step(t + 1);           // one step ahead
        if (t < NSTEP) {
#pragma unroll
          for (int eb = 0; eb < kPfEB; ++eb) acc[t & 1][eb] = mfma_fp8(av[t & 1], bfr[eb], floatx4{0.f, 0.f, 0.f, 0.f});
        }
        if (t > 0) {
          const int tp = t - 1, jp = tp / HBI, hbp = tp % HBI;
          const float4 w = wv[tp % 3];
          if (hbp == 0) {
#pragma unroll
            for (int eb = 0; eb < kPfEB; ++eb) part[eb] = g == jp ? lin[eb] : 0.f;
          }
#pragma unroll
          for (int eb = 0; eb < kPfEB; ++eb) {
            const floatx4 x = acc[tp & 1][eb];
            part[eb] = fmaf(w.x, fabsf(x[0]), part[eb]);
            part[eb] = fmaf(w.y, fabsf(x[1]), part[eb]);
            part[eb] = fmaf(w.z, fabsf(x[2]), part[eb]);
            part[eb] = fmaf(w.w, fabsf(x[3]), part[eb]);
          }
          if (hbp == HBI - 1) {
            // reduce-scatter over the 4 lane groups: lane group g ends with the totals of entry
            // blocks g and 4 + g for its column c16
            float h2[4];
#pragma unroll
            for (int p = 0; p < 4; ++p) {
              const auto x = __builtin_amdgcn_permlane16_swap(__float_as_uint(part[2 * p]),
                                                              __float_as_uint(part[2 * p + 1]), false, false);
              h2[p] = __uint_as_float(x[0]) + __uint_as_float(x[1]);
            }
            const auto y0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(h2[0]), __float_as_uint(h2[1]), false, false);
            const auto y1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(h2[2]), __float_as_uint(h2[3]), false, false);
            res0[jp] = (__uint_as_float(y0[0]) + __uint_as_float(y0[1])) * ks0 + 0.0f;
            res1[jp] = (__uint_as_float(y1[0]) + __uint_as_float(y1[1])) * ks1 + 0.0f;
          }
        }
        if (t > 0 && t < NSTEP) {
          // issue order within the step: the next step's LDS reads first (a whole step ahead of
          // their use), then one MFMA and four of the previous step's VALU, eight times.  Left
          // alone, the scheduler clusters the MFMAs (the in-order issue then serialises them with
          // the VALU work), pairs them with VALU reading their own fresh results, and sinks the
          // reads to the end of the step, just before their wait.
          if (t + 1 < NSTEP) __builtin_amdgcn_sched_group_barrier(0x100, 3, 0);
#pragma unroll
          for (int i = 0; i < kPfEB; ++i) {
            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
            __builtin_amdgcn_sched_group_barrier(0x002, 4, 0);
          }
        }
        __builtin_amdgcn_sched_barrier(0);             // steps do not mix
      }
#pragma unroll
      for (int j = 0; j < kPfQC; ++j) {
        float* srow = scores + ((int64_t)b * tb + (q_lo - t0) + s * kPfQC + j) * nsp;
        if (e_lo < nvq[j]) srow[e_lo] = res0[j];
        if (e_lo + 64 < nvq[j]) srow[e_lo + 64] = res1[j];
      }
    }
    if (s + 1 < nst) {
      LCS_PF_COMMIT((s + 1) & 1);   // that buffer was last read in stage s - 1, before the previous barrier
      __syncthreads();
    }
  }
#undef LCS_PF_FETCH
#undef LCS_PF_COMMIT
}

// 64-entry groups per wave in one decode scoring workgroup (4 waves): chunks of at most 4096 entries.
constexpr int kDecodeWaveGroups = 16;
constexpr int64_t kDecodeMaxChunk = 4 * kDecodeWaveGroups * 64;

// Decode scoring: one query row per workgroup, `chunk` entries per workgroup.  Loads return in order,
// so they are issued in the order they are needed: the query rows, then the chunk's key scales
// (staged in LDS), then each wave's first three 64-entry groups (they depend only on the chunk), so
// that the query preparation runs under the keys' latency: the 4 waves quantise one 16-head block
// each into LDS (codes + folded weights).  The chunk
// then streams in groups interleaved across waves, three groups in flight while the current group's
// 4*HBI MFMAs run back to back.  The epilogue applies relu and the head weights, reduce-scatters the
// 4 entry blocks over the 4 lane groups so that lane l ends with entry 64 gi + l, scales it, counts it
// in the LDS histogram and keeps it in LDS; the chunk's scores leave in one burst of 16-byte stores at
// the end.  Only key fragments are then in flight in the loop, so every wait is for a key group.
//
// NTK (fp8 keys): the keys are loaded non-temporally.  Chosen when the call's key stream is at least
// the Infinity Cache's size: such a stream cannot stay cached until the next step anyway, and
// loading it normally would evict what the step's other launches reuse (1M-token cache, batch 8:
// step 0.384 -> 0.379 ms).  Smaller streams load normally (a 128K-token cache, batch 32: the
// non-temporal loads made the call 0.0725 -> 0.077 ms).
template <bool FP8, int KS, int HBI, bool NTK>
__global__ void __launch_bounds__(256, (FP8 || KS * HBI <= 8) ? 2 : 1)
index_score_decode_kernel(const uint16_t* __restrict__ q_idx, const uint16_t* __restrict__ w_idx,
                          const void* __restrict__ ik, const float* __restrict__ ik_scale, int64_t ik_ld,
                          const int64_t* __restrict__ q_pos, int64_t n_cap, int Tq, int H_I, int dI, int m,
                          int64_t chunk, float* __restrict__ scores, uint32_t* __restrict__ hist, int64_t nsp) {
  typedef typename std::conditional<FP8, intx8, uint4>::type Frag;
  __shared__ uint32_t lhist[kBins];
  __shared__ Frag s_afr[HBI][KS][kWave];
  __shared__ float s_w[HBI * 16];
  __shared__ float s_sc[FP8 ? kDecodeMaxChunk : 1];     // the chunk's key scales
  __shared__ __align__(16) float s_sco[kDecodeMaxChunk];   // the chunk's scores

  const int lane = lane_id();
  // wave-uniform (readfirstlane): the group schedule below is then scalar control flow
  const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x / kWave);
  const int g = lane >> 4, c16 = lane & 15;
  const int64_t r = blockIdx.y;
  const int64_t b = r / Tq;
  const int64_t c0 = (int64_t)blockIdx.x * chunk;       // < n_cap: the grid covers the capacity
  const uint8_t* ik8 = static_cast<const uint8_t*>(ik) + b * ik_ld * dI;
  const uint16_t* ik16 = static_cast<const uint16_t*>(ik) + b * ik_ld * dI;
  const float* ksc = ik_scale ? ik_scale + b * ik_ld : nullptr;

  // Loads are unconditional (entry index clamped below `lim`) so that the compiler keeps them in
  // flight; the scores of out-of-range entries are never counted or read.
  auto load_group = [&](int64_t gi, int64_t lim, Frag (&fr)[4][KS]) {
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      int64_t e = c0 + 64 * gi + 16 * u + c16;
      e = e < lim ? e : lim - 1;
      if (FP8) {
        // bytes [16g, 16g + 16) and [64 + 16g, 64 + 16g + 16): each load instruction covers 64
        // contiguous bytes of 16 rows (the query codes use the same dim order)
        const intx4* p = reinterpret_cast<const intx4*>(ik8 + e * 128 + 16 * g);
        intx4 x0, x1;
        if constexpr (NTK) {
          x0 = __builtin_nontemporal_load(p);
          x1 = __builtin_nontemporal_load(p + 4);
        } else {
          x0 = p[0];
          x1 = p[4];
        }
        intx8 v = intx8{x0.x, x0.y, x0.z, x0.w, x1.x, x1.y, x1.z, x1.w};
        fr[u][0] = *reinterpret_cast<Frag*>(&v);
      } else {
#pragma unroll
        for (int ks = 0; ks < KS; ++ks) {
          uint4 v = *reinterpret_cast<const uint4*>(ik16 + e * dI + 32 * ks + 8 * g);
          fr[u][ks] = *reinterpret_cast<Frag*>(&v);
        }
      }
    }
  };

  // The query rows of the wave's head block come first (their wait then covers nothing else).
  const int head = wave * 16 + c16;
  const bool hv = wave < HBI && head < H_I;
  const int hl = hv ? head : H_I - 1;
  const uint16_t* qrow = q_idx + (r * H_I + hl) * dI;
  uint4 qraw[FP8 ? 4 : KS];
  uint32_t wraw = 0;
  if (wave < HBI) {
    if (FP8) {
      load_row_segments(qrow + 16 * g, qrow + 64 + 16 * g, *reinterpret_cast<uint4(*)[4]>(&qraw));
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) qraw[ks] = *reinterpret_cast<const uint4*>(qrow + 32 * ks + 8 * g);
    }
    wraw = w_idx[r * H_I + hl];
  }
  // Then the chunk's scales (one 256-entry slice per pass, thread t takes entry t of each) and the
  // first three groups of this wave (wave, wave + 4, wave + 8), clamped to the cache capacity: the row's
  // visible count is not known yet.  Entries past it are loaded in bounds and never counted; a wave
  // with fewer groups never computes the second buffer.
  constexpr int kScPasses = kDecodeMaxChunk / 256;
  const int64_t cl = c0 + chunk < n_cap ? c0 + chunk : n_cap;
  float scv[kScPasses];
  if (FP8) {
#pragma unroll
    for (int j = 0; j < kScPasses; ++j) {
      if (256 * j < chunk) {                              // uniform
        const int64_t e = c0 + 256 * j + threadIdx.x;
        scv[j] = ksc[e < cl ? e : cl - 1];
      }
    }
  }
  // key groups in flight ahead of the one computed: 3 (four buffers) where the registers allow
  // (fp8 keys, bf16 with dI = 64), else 2 (bf16 with dI = 128 would spill)
  constexpr int kAhead = (FP8 || KS <= 2) ? 3 : 2;
  Frag cur[4][KS], nxt[4][KS], nx2[4][KS], nx3[4][KS];
  load_group(wave, cl, cur);
  load_group(wave + 4, cl, nxt);
  if (kAhead == 3) load_group(wave + 8, cl, nx2);

  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  if (c0 >= nv) return;                                  // uniform
  const int64_t c1 = c0 + chunk < nv ? c0 + chunk : nv;

  for (int i = threadIdx.x; i < kBins; i += 256) lhist[i] = 0u;
  if (FP8) {
#pragma unroll
    for (int j = 0; j < kScPasses; ++j)
      if (256 * j < chunk) s_sc[256 * j + threadIdx.x] = scv[j];
  }
  if (wave < HBI) {
    // (an empty statement that takes the weight's bits: keeps their conversion, and so the wait for
    // them, here instead of right behind the load, ahead of the key loads)
    asm volatile("" : "+v"(wraw));
    float wh = hv ? bf2f((uint16_t)wraw) : 0.f;
    if (FP8) {
      intx8 codes;
      const float sc = quant_loaded_e4m3(*reinterpret_cast<const uint4(*)[4]>(&qraw), hv, codes);
      s_afr[wave][0][lane] = *reinterpret_cast<Frag*>(&codes);
      wh *= sc;
    } else {
#pragma unroll
      for (int ks = 0; ks < KS; ++ks) {
        const uint4 a = hv ? qraw[ks] : make_uint4(0, 0, 0, 0);
        s_afr[wave][ks][lane] = *reinterpret_cast<const Frag*>(&a);
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

  float* srow = scores + r * nsp;
  const int64_t ngroups = (c1 - c0 + 63) / 64;

  // Groups of this wave: wave + 4t, t = 0 .. nt-1.  kAhead + 1 register buffers rotate by unrolling
  // (a copy between buffers would wait for the loads in flight); kAhead groups stay in flight ahead of
  // the one being computed (fp8: two in flight measured 1.5-2 us slower per launch than three).
  // Loads past the end re-read the last group (never computed).
  const int64_t nt = ngroups > wave ? (ngroups - wave + 3) / 4 : 0;
  auto gidx = [&](int64_t t) -> int64_t { return wave + 4 * (t < nt ? t : nt - 1); };
  auto compute_group = [&](const Frag (&fr)[4][KS], int64_t gi) {
    // partial head sums of the lane's 4 heads per head block, entry column c16 of each row group u
    float p[4];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      floatx4 acc[HBI];
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
        acc[hb] = a;
      }
      float s = 0.f;
#pragma unroll
      for (int hb = 0; hb < HBI; ++hb)
#pragma unroll
        for (int i = 0; i < 4; ++i) s += wq[hb][i] * fmaxf(acc[hb][i], 0.f);
      p[u] = s;
    }
    // reduce-scatter over the lane groups: halves first (group g <-> g ^ 2), then rows (g <-> g ^ 1);
    // lane group g keeps row group u = g, i.e. lane l holds entry 64 gi + l
    const auto h0 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[0]), __float_as_uint(p[2]), false, false);
    const auto h1 = __builtin_amdgcn_permlane32_swap(__float_as_uint(p[1]), __float_as_uint(p[3]), false, false);
    const float r0 = __uint_as_float(h0[0]) + __uint_as_float(h0[1]);
    const float r1 = __uint_as_float(h1[0]) + __uint_as_float(h1[1]);
    const auto q01 = __builtin_amdgcn_permlane16_swap(__float_as_uint(r0), __float_as_uint(r1), false, false);
    const float tot = __uint_as_float(q01[0]) + __uint_as_float(q01[1]);
    const int j = (int)(64 * gi) + lane;                  // < chunk
    const float v = tot * (FP8 ? s_sc[j] : 1.f) + 0.0f;
    s_sco[j] = v;
    if (c0 + j < c1) atomicAdd(&lhist[float_key(v) >> kBinShift], 1u);
  };
  // Fully unrolled (nt <= kDecodeWaveGroups): straight-line code with forward exits only, so that
  // every wait for a group's loads leaves the three younger groups in flight (a loop back edge makes
  // the compiler's count of loads in flight conservative).
  if constexpr (kAhead == 3) {
#pragma unroll
    for (int t = 0; t < kDecodeWaveGroups; t += 4) {
      if (t >= nt) break;
      load_group(gidx(t + 3), c1, nx3);
      compute_group(cur, gidx(t));
      if (t + 1 >= nt) break;
      load_group(gidx(t + 4), c1, cur);
      compute_group(nxt, gidx(t + 1));
      if (t + 2 >= nt) break;
      load_group(gidx(t + 5), c1, nxt);
      compute_group(nx2, gidx(t + 2));
      if (t + 3 >= nt) break;
      load_group(gidx(t + 6), c1, nx2);
      compute_group(nx3, gidx(t + 3));
    }
  } else {
#pragma unroll
    for (int t = 0; t < kDecodeWaveGroups; t += 3) {
      if (t >= nt) break;
      load_group(gidx(t + 2), c1, nx2);
      compute_group(cur, gidx(t));
      if (t + 1 >= nt) break;
      load_group(gidx(t + 3), c1, cur);
      compute_group(nxt, gidx(t + 1));
      if (t + 2 >= nt) break;
      load_group(gidx(t + 4), c1, nxt);
      compute_group(nx2, gidx(t + 2));
    }
  }
  __syncthreads();
  // Scores [c0, c1) rounded up to a multiple of 4 entries: the rounding only reaches past the row's
  // visible end, within the row's stride (a multiple of 64), where readers mask by index.
  const int n4 = (int)((c1 - c0 + 3) >> 2);
  float4* dst = reinterpret_cast<float4*>(srow + c0);
  // (non-temporal: the scores are read once, by the selection launch)
  for (int i = threadIdx.x; i < n4; i += 256)
    __builtin_nontemporal_store(reinterpret_cast<const floatx4*>(s_sco)[i], reinterpret_cast<floatx4*>(dst) + i);
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
  const uint32_t incl = wave_incl_scan(v);
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

__device__ __forceinline__ int final_slot(int i) { return (i % kFinalSeg) * kFinalStride + i / kFinalSeg; }

struct FinalShared {
  unsigned long long list[kFinalSeg * kFinalStride];
  uint32_t keep[kMaxDecodeChunks];   // kept entries per chunk
  uint32_t pos[kMaxDecodeChunks];    // their offset in the concatenated list / in the output
  uint32_t h[256];
  unsigned long long prefix;
  int remaining, done, shift, T2, above2;
};

// Row r's selection (the row's visible entries: n_visible of its query position).
__device__ __forceinline__ void final_select(FinalShared& sh, uint32_t* s_w, int64_t r, const int64_t* q_pos, int m,
                                             int64_t n_cap, const unsigned long long* __restrict__ comb,
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
  const unsigned long long* lrow = comb + r * nsp;

  // ---- one round trip, issued with the query position's load rather than after it (every
  //      address is clamped into the row's regions, not to its visible part): the per-chunk counts
  //      and, speculatively, the first 64 list entries of each of the first 64 chunks (wave w:
  //      chunks w, w + 4, ...), which usually hold the whole list ----
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  constexpr int kHeadChunks = kWaves * 16;
  unsigned long long vh[16];
#pragma unroll
  for (int u = 0; u < 16; ++u) {
    const int c = min(wave + kWaves * u, nchunk - 1);
    vh[u] = lrow[min((int64_t)c * kFilterChunk + lane, nsp - 1)];
  }
  const uint32_t* h2 = hist + r * kHistRow + kBins;
  const uint4 h2a = *reinterpret_cast<const uint4*>(h2 + tid * 8);
  const uint4 h2b = *reinterpret_cast<const uint4*>(h2 + tid * 8 + 4);
  constexpr int kPerT = kMaxDecodeChunks / kSelThreads;   // 8
  uint2 ccv[kPerT];
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = tid * kPerT + u;
    ccv[u] = counts[r * nchunk + (c < nchunk ? c : 0)];
  }
  if (nv <= k) {                                    // every visible entry, ascending
    for (int64_t i = tid; i < k; i += kSelThreads) {
      out[i] = i < nv ? (int32_t)i : -1;
      if (out_s) out_s[i] = i < nv ? srow[i] : -INFINITY;
    }
    return;
  }
  const int nch = (int)((nv + kFilterChunk - 1) / kFilterChunk);
  const bool heads = nch <= kHeadChunks;
  uint32_t kc[kPerT];
  uint32_t ksum = 0, asum = 0;
#pragma unroll
  for (int u = 0; u < kPerT; ++u) {
    const int c = tid * kPerT + u;
    kc[u] = c < nch ? ccv[u].x : 0u;
    ksum += kc[u];
    asum += c < nch ? ccv[u].y : 0u;
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
        const uint32_t incl = wave_incl_scan(lsum);
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
  const int64_t c0 = (int64_t)blockIdx.x * kFilterChunk;
  constexpr int kPer = kFilterChunk / kSelThreads;           // 16 consecutive entries per thread
  const int64_t e0 = c0 + (int64_t)kPer * tid;
  const float* srow = scores + r * nsp;
  // the score loads go out with the query position's load, not after it: they are clamped into the
  // row's region (nsp is a multiple of 64), and entries past the visible ones are masked below
  const int64_t q4max = (nsp >> 2) - 1;
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const uint32_t* hrow = hist + r * kHistRow;               // the row histogram, first back
  const uint4 ha = *reinterpret_cast<const uint4*>(hrow + tid * 8);
  const uint4 hb = *reinterpret_cast<const uint4*>(hrow + tid * 8 + 4);
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
  if (c0 >= nv) return;                                      // uniform
  if (tid == 0) { sT = -1; sAbove = 0; }
  __syncthreads();
  if (nv > k) {
    const uint32_t loc[8] = {ha.x, ha.y, ha.z, ha.w, hb.x, hb.y, hb.z, hb.w};
    find_threshold_bins(loc, k, &sT, &sAbove, s_w);
  }
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

// Decode final: one workgroup per row runs the selection above, then clears the row's histograms
// (both levels; nothing reads them after this kernel in the call) for the next call.
__global__ void __launch_bounds__(kSelThreads)
topk_final_kernel(const unsigned long long* __restrict__ comb, const uint2* __restrict__ counts,
                  uint32_t* __restrict__ hist, int64_t nsp, int nchunk, const int64_t* __restrict__ q_pos,
                  int m, int64_t n_cap, int k, const float* __restrict__ scores, int32_t* __restrict__ topk_idx,
                  float* __restrict__ topk_score) {
  __shared__ FinalShared sh;
  __shared__ uint32_t s_w[kSelThreads / kWave];
  const int64_t r = blockIdx.x;
  final_select(sh, s_w, r, q_pos, m, n_cap, comb, counts, hist, nsp, nchunk, k, scores, topk_idx, topk_score);
  __syncthreads();                                // every read of the level-2 histogram is done
  uint4* h = reinterpret_cast<uint4*>(hist + r * kHistRow);
  for (int i = threadIdx.x; i < kHistRow / 4; i += kSelThreads) h[i] = make_uint4(0u, 0u, 0u, 0u);
}

// The final selection with a decode token append beside it: workgroups x < R select row x, the
// next B run the append of sequence x - R on their first 128 threads.  The two touch disjoint
// buffers (the selection's workspace and output; the append's state, ring and caches), and nothing
// the append writes is read by this call's selection: the entry a token finishes lies past the
// visible range of a query at that token.  One launch fewer per CSA decode layer.
__global__ void __launch_bounds__(kSelThreads)
topk_final_append_kernel(const unsigned long long* __restrict__ comb, const uint2* __restrict__ counts,
                         uint32_t* __restrict__ hist, int64_t nsp, int nchunk, const int64_t* __restrict__ q_pos,
                         int m, int64_t n_cap, int k, const float* __restrict__ scores, int32_t* __restrict__ topk_idx,
                         float* __restrict__ topk_score, int R, DecodeAppendArgs ap, RopeFreq rf) {
  __shared__ FinalShared sh;
  __shared__ uint32_t s_w[kSelThreads / kWave];
  __shared__ float red[2];
  if ((int)blockIdx.x >= R) {
    if (threadIdx.x >= dapp::kThreads) return;       // whole waves: the append's barriers count the rest
    dapp::decode_append_seq(ap, rf, (int)blockIdx.x - R, red);
    return;
  }
  const int64_t r = blockIdx.x;
  final_select(sh, s_w, r, q_pos, m, n_cap, comb, counts, hist, nsp, nchunk, k, scores, topk_idx, topk_score);
  __syncthreads();                                // every read of the level-2 histogram is done
  uint4* h = reinterpret_cast<uint4*>(hist + r * kHistRow);
  for (int i = threadIdx.x; i < kHistRow / 4; i += kSelThreads) h[i] = make_uint4(0u, 0u, 0u, 0u);
}

constexpr int kCandCache = 4096;            // candidate keys kept in LDS during the digit passes
constexpr int kSampleBlock = 32;            // sampled run of consecutive entries (one 128-byte line)
constexpr int kSampleBlocks = 512;          // sampled runs per row, at most
constexpr int kSampleMinStride = 512;       // at least 16x fewer lines than the row
constexpr int64_t kSampleMinRow = 8192;     // shorter rows take the full path
constexpr int kSampleMinRatio = 8;          // ... and rows with k above an eighth of them
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

// Resolve `need` winners among `ncand` candidate keys digit by digit and append their entry indices
// to sel_list.  A key is `key_bits` wide: the score-key bits (all 32, or the 21 below a common bin),
// then the complemented entry index (32 bits).  Keys are read once into LDS when they fit.
// in_lds: the candidates are already in s.u.ckey (ncand <= kCandCache), cand is not read.
__device__ __forceinline__ void refine_candidates(const unsigned long long* cand, int ncand, int need, int32_t* sel_list,
                                  SelShared& s, int key_bits = 53, bool in_lds = false) {
  const int tid = threadIdx.x;
  const bool cached = ncand <= kCandCache;
  if (cached && !in_lds) {               // all loads first, then the LDS stores (one round trip)
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
  int shift = key_bits;
  for (int pass = 0; pass < 8 && shift > 0; ++pass) {
    const int width = shift >= 8 ? 8 : shift;
    shift -= width;
    for (int i = tid; i < 256; i += kSelThreads) s.h256[i] = 0u;
    __syncthreads();
    const unsigned long long pre = s.prefix;
    const int hi = shift + width;                 // 64 on the first pass of 64-bit keys: every key matches
    auto match = [&](uint64_t key) { return hi >= 64 || (key >> hi) == pre; };
    if (cached) {
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint64_t key = s.u.ckey[i];
        if (match(key)) atomicAdd(&s.h256[(key >> shift) & ((1u << width) - 1u)], 1u);
      }
    } else {
      for (int i = tid; i < ncand; i += kSelThreads) {
        const uint64_t key = src[i];
        if (match(key)) atomicAdd(&s.h256[(key >> shift) & ((1u << width) - 1u)], 1u);
      }
    }
    __syncthreads();
    if (tid < kWave) {
      // lane j covers digits 255-4j .. 252-4j (top first)
      uint32_t c[4];
      uint32_t lsum = 0;
#pragma unroll
      for (int u = 0; u < 4; ++u) { c[u] = s.h256[255 - 4 * tid - u]; lsum += c[u]; }
      const uint32_t incl = wave_incl_scan(lsum);
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
    const uint32_t incl = wave_incl_scan(cnt);
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

// Prefill rows of at most kWaveRowMax visible entries: one wave per row, no workgroup barrier.  The
// wave holds the row's order-preserving keys in registers (lane l: entries 16 l .. 16 l + 15; past the
// row: key 0, below every finite score's key), finds the k-th largest key by four 8-bit radix passes
// (a 256-bin LDS histogram of its own, scanned from the top by the lanes four bins each), and writes
// the keys above it plus the lowest-index keys equal to it, in index order.
constexpr int kWaveRowMax = 1024;
constexpr int kWaveRowPer = kWaveRowMax / kWave;    // 16 keys per lane
constexpr int kWaveRowWaves = 4;                    // rows per workgroup

// The wave's earlier LDS accesses are complete before its later ones (the histogram is the wave's own).
__device__ __forceinline__ void wave_lds_order() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

__global__ void __launch_bounds__(kWaveRowWaves * kWave)
topk_wave_kernel(const float* __restrict__ scores, int64_t nsp, const int64_t* __restrict__ q_pos, int m,
                 int64_t n_cap, int k, int Tq, int t0, int tcur, int tb, int nrows, int32_t* __restrict__ topk_idx,
                 float* __restrict__ topk_score) {
  __shared__ __align__(16) uint32_t hist[kWaveRowWaves][256];
  const int lane = lane_id();
  const int wv = threadIdx.x / kWave;
  const int x = blockIdx.x * kWaveRowWaves + wv;      // row x of this batch: (x / tcur, t0 + x % tcur)
  if (x >= nrows) return;                              // wave-uniform
  const int64_t bq = x / tcur, tq = t0 + x % tcur;
  const int64_t r = bq * Tq + tq;
  const int64_t rb = bq * tb + (tq - t0);
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const float* srow = scores + rb * nsp;
  int32_t* oi = topk_idx + r * k;
  float* os = topk_score ? topk_score + r * k : nullptr;
  if (nv <= k) {
    for (int i = lane; i < k; i += kWave) {
      oi[i] = i < nv ? i : -1;
      if (os) os[i] = i < nv ? srow[i] : -INFINITY;
    }
    return;
  }
  // entries 16 lane + j, read inside the row (nsp >= 64 is a multiple of 64)
  const int64_t e0 = 16 * lane;
  const float4* src = reinterpret_cast<const float4*>(srow + (e0 + 16 <= nsp ? e0 : nsp - 16));
  float val[kWaveRowPer];
#pragma unroll
  for (int q = 0; q < kWaveRowPer / 4; ++q) {
    const float4 v = src[q];
    val[4 * q] = v.x; val[4 * q + 1] = v.y; val[4 * q + 2] = v.z; val[4 * q + 3] = v.w;
  }
  uint32_t key[kWaveRowPer];
#pragma unroll
  for (int j = 0; j < kWaveRowPer; ++j) key[j] = e0 + j < nv ? float_key(val[j]) : 0u;

  uint32_t* hw = hist[wv];
  uint32_t prefix = 0u, pmask = 0u;
  uint32_t kk = (uint32_t)k;               // rank, from the top, of the k-th key among those matching prefix
#pragma unroll
  for (int pass = 0; pass < 4; ++pass) {
    const int sh = 24 - 8 * pass;
    reinterpret_cast<uint4*>(hw)[lane] = make_uint4(0u, 0u, 0u, 0u);
    wave_lds_order();
#pragma unroll
    for (int j = 0; j < kWaveRowPer; ++j)
      if ((key[j] & pmask) == prefix) atomicAdd(&hw[(key[j] >> sh) & 255u], 1u);
    wave_lds_order();
    uint32_t c[4];                         // bins 255 - 4 lane - q, descending
#pragma unroll
    for (int q = 0; q < 4; ++q) c[q] = hw[255 - 4 * lane - q];
    wave_lds_order();
    const uint32_t s4 = c[0] + c[1] + c[2] + c[3];
    const uint32_t incl = wave_incl_scan(s4);
    const uint32_t excl = incl - s4;
    const bool here = excl < kk && kk <= incl;
    const uint64_t bl = __ballot(here);
    const int srcl = bl ? __ffsll((unsigned long long)bl) - 1 : 0;
    int bin = 0;
    uint32_t above = excl;
    if (here) {
      bin = 252 - 4 * lane;
      bool found = false;
#pragma unroll
      for (int q = 0; q < 4; ++q) {
        if (!found && above + c[q] >= kk) { bin = 255 - 4 * lane - q; found = true; }
        else if (!found) above += c[q];
      }
    }
    bin = __builtin_amdgcn_readlane(bin, srcl);
    above = (uint32_t)__builtin_amdgcn_readlane((int)above, srcl);
    prefix |= (uint32_t)bin << sh;
    pmask |= 255u << sh;
    kk -= above;
  }
  // prefix is the k-th largest key; every key above it and the kk lowest-index keys equal to it win
  uint32_t eq = 0u, gt = 0u;
#pragma unroll
  for (int j = 0; j < kWaveRowPer; ++j) {
    eq += key[j] == prefix ? 1u : 0u;
    gt += key[j] > prefix ? 1u : 0u;
  }
  const uint32_t eq_before = wave_incl_scan(eq) - eq;
  const uint32_t take_eq = kk > eq_before ? (kk - eq_before < eq ? kk - eq_before : eq) : 0u;
  const uint32_t cnt = gt + take_eq;
  uint32_t pos = wave_incl_scan(cnt) - cnt;
  uint32_t er = eq_before;
#pragma unroll
  for (int j = 0; j < kWaveRowPer; ++j) {
    const bool tie = key[j] == prefix;
    const bool win = key[j] > prefix || (tie && er < kk);
    er += tie ? 1u : 0u;
    if (win && pos < (uint32_t)k) {        // exactly k win; the bound keeps every store in the row
      oi[pos] = (int32_t)(e0 + j);
      if (os) os[pos] = val[j];
      ++pos;
    }
  }
}

// Prefill: one workgroup per row does histogram, filter, refine, sort.
__global__ void __launch_bounds__(kSelThreads)
topk_rowwise_kernel(const float* __restrict__ scores, unsigned long long* __restrict__ cand, int64_t nsp,
                    const int64_t* __restrict__ q_pos, int m, int64_t n_cap, int k, int Tq, int t0, int tcur,
                    int tb, int32_t* __restrict__ topk_idx, float* __restrict__ topk_score) {
  __shared__ SelShared s;
  __shared__ int32_t list[kMaxTopk];
  __shared__ __align__(16) uint32_t h[kBins];
  __shared__ int sT, sAbove, sCand;
  const int tid = threadIdx.x;
  // workgroup x: query position t0 + x % tcur of batch row x / tcur (buffer row b * tb + x % tcur)
  const int64_t bq = blockIdx.x / tcur, tq = t0 + blockIdx.x % tcur;
  const int64_t r = bq * Tq + tq;
  const int64_t rb = bq * tb + (tq - t0);
  const int64_t nv = n_visible(q_pos, r, m, n_cap);
  const float* srow = scores + rb * nsp;
  if (nv <= k) {
    for (int64_t i = tid; i < k; i += kSelThreads) {
      topk_idx[r * k + i] = i < nv ? (int32_t)i : -1;
      if (topk_score) topk_score[r * k + i] = i < nv ? srow[i] : -INFINITY;
    }
    return;
  }
  unsigned long long* crow = cand + rb * nsp;
  // ---- Sampled threshold (long rows, k a small fraction): a lower bound on the k-th key from a
  // sample of whole 32-entry blocks, then a single pass keeps every entry at or above it.  Exact
  // whenever at least k entries pass (the k winners are then all among them); else the full path.
  if (nv >= kSampleMinRow && nv >= (int64_t)kSampleMinRatio * k) {
    int64_t stride = (nv + kSampleBlocks - 1) / kSampleBlocks;
    stride = stride < kSampleMinStride ? kSampleMinStride : (stride + kSampleBlock - 1) / kSampleBlock * kSampleBlock;
    const int64_t nblk = (nv - kSampleBlock) / stride + 1;     // blocks b * stride + [0, 32), all < nv
    const int S = (int)(nblk * kSampleBlock);
    const double expect = (double)k * S / (double)nv;        // sample entries expected above the k-th
    const int j = (int)ceil(expect + 3.0 * sqrt(expect) + 8.0);
    if (j <= S / 2) {
      // the thread's sample keys (entries tid + 256 u), all loads in flight at once, kept in registers
      // for both histogram levels
      constexpr int kSampPer = kSampleBlocks * kSampleBlock / kSelThreads;   // 64
      uint32_t sk[kSampPer];
#pragma unroll
      for (int u = 0; u < kSampPer; ++u) {
        const int i = tid + kSelThreads * u;
        const int ic = i < S ? i : 0;                         // a readable entry
        sk[u] = float_key(srow[(ic / kSampleBlock) * stride + ic % kSampleBlock]);
      }
      for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0u;
      if (tid == 0) { sT = -1; sAbove = 0; sCand = 0; s.nsel = 0; }
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kSampPer; ++u)
        if (tid + kSelThreads * u < S) atomicAdd(&h[sk[u] >> kBinShift], 1u);
      __syncthreads();
      find_threshold(h, j, &sT, &sAbove, s.scan);          // bin of the sample's j-th largest key
      const int T1 = sT, rem = j - sAbove;
      for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0u;
      __syncthreads();
#pragma unroll
      for (int u = 0; u < kSampPer; ++u)
        if (tid + kSelThreads * u < S && (int)(sk[u] >> kBinShift) == T1)
          atomicAdd(&h[(sk[u] >> (kBinShift - 11)) & (kBins - 1)], 1u);
      __syncthreads();
      find_threshold(h, rem, &sT, &sAbove, s.scan);        // ... refined by its next 11 bits
      const uint32_t thr = ((uint32_t)T1 << kBinShift) | ((uint32_t)sT << (kBinShift - 11));
      // one pass: 16 consecutive entries per thread per round, wave-aggregated appends.  The loads
      // are unconditional (clamped into the row's buffer, entries past nv masked after) and the
      // next round's are in flight while a round is filtered (two register sets, alternating).
      const int lane = lane_id();
      constexpr int64_t kRound = 16 * kSelThreads;
      auto load16 = [&](int64_t e0, float4& x0, float4& x1, float4& x2, float4& x3) {
        int64_t eb = e0 + 16 * tid;
        eb = eb < nsp - 16 ? eb : nsp - 16;                // readable: nsp is a multiple of 64
        const float4* p = reinterpret_cast<const float4*>(srow + eb);
        x0 = p[0]; x1 = p[1]; x2 = p[2]; x3 = p[3];
      };
      // TO_LDS: candidates go to the refine phase's LDS key array (positions past it are counted, not
      // stored), so the pass's memory counter holds only its loads; else to the row's global list
      auto filter16 = [&](auto to_lds_c, int64_t e0, const float4& x0, const float4& x1, const float4& x2,
                          const float4& x3) {
        constexpr bool kToLds = decltype(to_lds_c)::value;
        const int64_t eb = e0 + 16 * tid;
        const float4 xs[4] = {x0, x1, x2, x3};
        uint32_t keys[16];
#pragma unroll
        for (int q = 0; q < 4; ++q) {
          keys[4 * q] = float_key(xs[q].x); keys[4 * q + 1] = float_key(xs[q].y);
          keys[4 * q + 2] = float_key(xs[q].z); keys[4 * q + 3] = float_key(xs[q].w);
        }
        uint32_t keep = 0;
#pragma unroll
        for (int i = 0; i < 16; ++i) keep |= (eb + i < nv && keys[i] >= thr ? 1u : 0u) << i;
        if (__ballot(keep != 0u) == 0ull) return;             // wave-uniform: nothing kept
        const uint32_t c = (uint32_t)__popc(keep);
        const uint32_t incl = wave_incl_scan(c);
        uint32_t base = 0;
        if (lane == kWave - 1) base = (uint32_t)atomicAdd(&sCand, (int)incl);
        base = __shfl(base, kWave - 1, kWave) + incl - c;
#pragma unroll
        for (int i = 0; i < 16; ++i)
          if ((keep >> i) & 1u) {
            const unsigned long long v = ((unsigned long long)keys[i] << 32) | (unsigned long long)(0xFFFFFFFFu - (uint32_t)(eb + i));
            if (kToLds) {
              if (base < (uint32_t)kCandCache) s.u.ckey[base] = v;
            } else {
              crow[base] = v;
            }
            ++base;
          }
      };
      auto run_pass = [&](auto to_lds_c) {
        float4 a0, a1, a2, a3, b0, b1, b2, b3;
        load16(0, a0, a1, a2, a3);
        for (int64_t e0 = 0; e0 < nv; e0 += 2 * kRound) {
          load16(e0 + kRound, b0, b1, b2, b3);
          __builtin_amdgcn_sched_barrier(0);               // the next round's loads go out first
          filter16(to_lds_c, e0, a0, a1, a2, a3);
          if (e0 + kRound >= nv) break;                     // uniform
          load16(e0 + 2 * kRound, a0, a1, a2, a3);
          __builtin_amdgcn_sched_barrier(0);
          filter16(to_lds_c, e0 + kRound, b0, b1, b2, b3);
        }
      };
      run_pass(std::true_type{});
      __syncthreads();
      int ncand = sCand;
      bool in_lds = true;
      if (ncand > kCandCache) {                             // uniform, rare: the pass again, to HBM
        __syncthreads();                                    // every thread has read sCand
        if (tid == 0) sCand = 0;
        __syncthreads();
        run_pass(std::false_type{});
        __syncthreads();
        ncand = sCand;
        in_lds = false;
      }
      if (ncand >= k) {                                    // uniform
        refine_candidates(crow, ncand, k, list, s, 64, in_lds);
        sort_and_write(list, k, nv, k, srow, topk_idx + r * k, topk_score ? topk_score + r * k : nullptr, s);
        return;
      }
      __syncthreads();                                     // the full path reuses h and the counters
    }
  }
  for (int i = tid; i < kBins; i += kSelThreads) h[i] = 0u;
  if (tid == 0) { s.nsel = 0; sCand = 0; sT = kBins - 1; sAbove = 0; }
  __syncthreads();
  for (int64_t e = tid; e < nv; e += kSelThreads) atomicAdd(&h[float_key(srow[e]) >> kBinShift], 1u);
  __syncthreads();
  find_threshold(h, k, &sT, &sAbove, s.scan);
  const int T = sT;
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

// Entries per decode scoring workgroup: about two workgroups per CU over the whole call, at most
// kDecodeMaxChunk (larger calls take more workgroups).
int64_t decode_chunk(int64_t n_cap, int R) {
  int64_t c = (n_cap * R + 511) / 512;
  c = (c + 255) & ~(int64_t)255;
  if (c < 256) c = 256;
  if (c > kDecodeMaxChunk) c = kDecodeMaxChunk;
  return c;
}

constexpr int64_t kInfinityCacheBytes = (int64_t)256 << 20;   // MI355X's memory-side cache

template <bool FP8, int KS, int HBI>
void launch_score_decode(const IndexArgs& a, const Ws& w, hipStream_t st) {
  const int64_t chunk = decode_chunk(a.n_cap, a.B * a.Tq);
  dim3 grid((unsigned)((a.n_cap + chunk - 1) / chunk), (unsigned)(a.B * a.Tq));
  // key bytes the call streams (codes and row scales of every entry of every row's capacity)
  const bool ntk = (int64_t)a.B * a.Tq * a.n_cap * (a.dI + 4) >= kInfinityCacheBytes;
  if constexpr (FP8) {
    if (ntk) {
      LCS_LAUNCH("index_score_kernel", (index_score_decode_kernel<FP8, KS, HBI, true>), grid, dim3(256), 0, st,
                 a.q_idx, a.w_idx, a.ik, a.ik_scale, a.ik_ld, a.q_pos, a.n_cap, a.Tq, a.H_I, a.dI, a.m, chunk,
                 w.scores, w.hist, w.nsp);
      return;
    }
  }
  LCS_LAUNCH("index_score_kernel", (index_score_decode_kernel<FP8, KS, HBI, false>), grid, dim3(256), 0, st,
             a.q_idx, a.w_idx, a.ik, a.ik_scale, a.ik_ld, a.q_pos, a.n_cap, a.Tq, a.H_I, a.dI, a.m, chunk,
             w.scores, w.hist, w.nsp);
}

template <int KS, int HBI>
void launch_score_rows_bf16(const IndexArgs& a, const Ws& w, int t0, int tcur, int tb, hipStream_t st) {
  const int tiles = (tcur + 15) / 16;
  // entries per workgroup: kScoreChunk, halved (down to 64) while the grid has fewer than about 1024
  // workgroups (short caches: a 1024-entry chunk per 16 queries leaves most CUs idle)
  int chunk = kScoreChunk;
  while (chunk > 64 && ((a.n_cap + chunk - 1) / chunk) * a.B * tiles < 1024) chunk /= 2;
  dim3 grid((unsigned)((a.n_cap + chunk - 1) / chunk), (unsigned)(a.B * tiles));
  LCS_LAUNCH("index_score_kernel", (index_score_kernel<KS, HBI>), grid, dim3(256), 0, st, a.q_idx, a.w_idx,
             static_cast<const uint16_t*>(a.ik), a.ik_ld, a.q_pos, a.n_cap, a.Tq, t0, tcur, tb, a.H_I, a.dI, a.m,
             w.scores, w.nsp, chunk);
}

// fp8 prefill grid: one workgroup per chunk of kPfChunk entries (x) and per query range of each
// batch row (y); the query ranges (multiples of kPfQC) are split so that there are enough
// workgroups for two per CU when the chunks alone are fewer.
struct PfGrid {
  int64_t nchunk;
  int qsplit, qper;
};
PfGrid prefill_grid(int B, int Tq, int64_t n_cap) {
  PfGrid p;
  p.nchunk = (n_cap + kPfChunk - 1) / kPfChunk;
  const int nstage = (Tq + kPfQC - 1) / kPfQC;
  const int64_t want = (512 + p.nchunk * B - 1) / (p.nchunk * B);
  const int qs0 = (int)(want < nstage ? want : nstage);
  p.qper = (nstage + qs0 - 1) / qs0 * kPfQC;
  p.qsplit = (Tq + p.qper - 1) / p.qper;
  return p;
}

template <int HBI>
void launch_qprep_fp8(const IndexArgs& a, const Ws& w, hipStream_t st) {
  LCS_LAUNCH("index_qprep_kernel", index_qprep_kernel<HBI>, dim3((unsigned)(a.B * a.Tq)), dim3(256), 0, st,
             a.q_idx, a.w_idx, a.H_I, a.q_pos, a.n_cap, a.m, a.Tq, w.qc, w.qw, w.qnv, w.linc, w.lins);
}
template <int HBI>
void launch_score_rows_fp8(const IndexArgs& a, const Ws& w, int t0, int tcur, int tb, hipStream_t st) {
  const PfGrid p = prefill_grid(a.B, tcur, a.n_cap);
  dim3 grid((unsigned)p.nchunk, (unsigned)(a.B * p.qsplit));
  LCS_LAUNCH("index_score_kernel", index_score_prefill_kernel<HBI>, grid, dim3(kPfWaves * kWave), 0, st, w.qc, w.qw,
             w.qnv, w.linc, w.lins, static_cast<const uint8_t*>(a.ik), a.ik_scale, a.ik_ld, a.n_cap, a.Tq, t0, tcur,
             tb, p.qsplit, p.qper, w.scores, w.nsp);
}

void score_decode(const IndexArgs& a, const Ws& w, hipStream_t st) {
  const int hbi = (a.H_I + 15) / 16;
  if (a.ik_fp8) {
    if (hbi == 1) launch_score_decode<true, 1, 1>(a, w, st);
    else if (hbi == 2) launch_score_decode<true, 1, 2>(a, w, st);
    else launch_score_decode<true, 1, 4>(a, w, st);
  } else if (a.dI == 64) {
    if (hbi == 1) launch_score_decode<false, 2, 1>(a, w, st);
    else if (hbi == 2) launch_score_decode<false, 2, 2>(a, w, st);
    else launch_score_decode<false, 2, 4>(a, w, st);
  } else {
    if (hbi == 1) launch_score_decode<false, 4, 1>(a, w, st);
    else if (hbi == 2) launch_score_decode<false, 4, 2>(a, w, st);
    else launch_score_decode<false, 4, 4>(a, w, st);
  }
}

// fp8: the query rows' codes, weights and linear terms, once for all rows
void prep_rows(const IndexArgs& a, const Ws& w, hipStream_t st) {
  if (!a.ik_fp8) return;
  const int hbi = (a.H_I + 15) / 16;
  if (hbi == 1) launch_qprep_fp8<1>(a, w, st);
  else if (hbi == 2) launch_qprep_fp8<2>(a, w, st);
  else if (hbi == 3) launch_qprep_fp8<3>(a, w, st);
  else launch_qprep_fp8<4>(a, w, st);
}

// scores of query positions [t0, t0 + tcur) of every batch row into buffer rows b * tb + (t - t0)
void score_rows(const IndexArgs& a, const Ws& w, int t0, int tcur, int tb, hipStream_t st) {
  const int hbi = (a.H_I + 15) / 16;
  if (a.ik_fp8) {
    if (hbi == 1) launch_score_rows_fp8<1>(a, w, t0, tcur, tb, st);
    else if (hbi == 2) launch_score_rows_fp8<2>(a, w, t0, tcur, tb, st);
    else if (hbi == 3) launch_score_rows_fp8<3>(a, w, t0, tcur, tb, st);
    else launch_score_rows_fp8<4>(a, w, t0, tcur, tb, st);
  } else if (a.dI == 64) {
    if (hbi == 1) launch_score_rows_bf16<2, 1>(a, w, t0, tcur, tb, st);
    else if (hbi == 2) launch_score_rows_bf16<2, 2>(a, w, t0, tcur, tb, st);
    else launch_score_rows_bf16<2, 4>(a, w, t0, tcur, tb, st);
  } else {
    if (hbi == 1) launch_score_rows_bf16<4, 1>(a, w, t0, tcur, tb, st);
    else if (hbi == 2) launch_score_rows_bf16<4, 2>(a, w, t0, tcur, tb, st);
    else launch_score_rows_bf16<4, 4>(a, w, t0, tcur, tb, st);
  }
}

}  // namespace

// Every grid the call would launch fits the HIP limits (x < 2^31, y <= 65535).
bool index_topk_launchable(int B, int Tq, int64_t n_cap, int ik_fp8) {
  const int64_t R = (int64_t)B * Tq;
  if (R < kDecodeRows && n_chunks(n_cap) <= kMaxDecodeChunks) return true;   // decode grids (chunks, R)
  if (R >= ((int64_t)1 << 31)) return false;                         // one workgroup per row
  const int tb = prefill_batch(B, Tq, n_cap);          // query positions per batch launch
  if ((int64_t)B * tb >= ((int64_t)1 << 31)) return false;
  if (ik_fp8) {
    const PfGrid p = prefill_grid(B, tb, n_cap);
    return p.nchunk < ((int64_t)1 << 31) && (int64_t)B * p.qsplit <= 65535;
  }
  return (n_cap + 63) / 64 < ((int64_t)1 << 31) && (int64_t)B * ((tb + 15) / 16) <= 65535;
}

size_t index_topk_state_bytes() { return al256((size_t)kDecodeRows * kHistRow * 4); }

size_t index_topk_workspace(int B, int Tq, int64_t n_cap, int k) {
  (void)k;
  const int64_t R = (int64_t)B * Tq;
  const int64_t RS = buffer_rows(B, Tq, n_cap);
  const int64_t nsp = (n_cap + 63) & ~(int64_t)63;
  return al256((size_t)kDecodeRows * kHistRow * 4) + al256((size_t)RS * nsp * 4) + al256((size_t)RS * nsp * 8) +
         al256((size_t)R * n_chunks(n_cap) * 8) + al256((size_t)R * kMaxIndexHeads * 128) +
         al256((size_t)R * kMaxIndexHeads * 4) + al256((size_t)R * 4) + al256((size_t)n_groups4(B, Tq) * 2048) +
         al256((size_t)n_groups4(B, Tq) * 256);
}

int launch_index_topk(const IndexArgs& a, hipStream_t st) {
  const int R = a.B * a.Tq;
  Ws w = carve(a.ws, a.B, a.Tq, a.n_cap);
  // Few rows: spread every row over many workgroups (decode).  Many rows, or rows longer than the
  // decode selection stages: row-per-workgroup.
  const bool decode = decode_rows(a.B, a.Tq, a.n_cap);
  if (decode) {
    score_decode(a, w, st);                       // the histogram rows start at zero (see kDecodeRows)
    dim3 gf((unsigned)w.nchunk, (unsigned)R);
    LCS_LAUNCH("topk_filter_kernel", topk_filter_kernel, gf, dim3(kSelThreads), 0, st, w.scores, w.hist, w.comb,
               w.counts, w.nsp, w.nchunk, a.q_pos, a.m, a.n_cap, a.k);
    if (a.append) {
      LCS_LAUNCH("topk_final_kernel", topk_final_append_kernel, dim3((unsigned)(R + a.append->B)), dim3(kSelThreads),
                 0, st, w.comb, w.counts, w.hist, w.nsp, w.nchunk, a.q_pos, a.m, a.n_cap, a.k, w.scores, a.topk_idx,
                 a.topk_score, R, *a.append, rope_freq(a.append->theta));
    } else {
      LCS_LAUNCH("topk_final_kernel", topk_final_kernel, dim3((unsigned)R), dim3(kSelThreads), 0, st, w.comb,
                 w.counts, w.hist, w.nsp, w.nchunk, a.q_pos, a.m, a.n_cap, a.k, w.scores, a.topk_idx, a.topk_score);
    }
  } else {
    // batches of query positions: score, then select, reusing the score and candidate buffers
    prep_rows(a, w, st);
    const int tb = prefill_batch(a.B, a.Tq, a.n_cap);
    for (int t0 = 0; t0 < a.Tq; t0 += tb) {
      const int tcur = a.Tq - t0 < tb ? a.Tq - t0 : tb;
      score_rows(a, w, t0, tcur, tb, st);
      if (a.n_cap <= kWaveRowMax) {            // short rows: one wave each
        const int nrows = a.B * tcur;
        LCS_LAUNCH("topk_wave_kernel", topk_wave_kernel, dim3((unsigned)((nrows + kWaveRowWaves - 1) / kWaveRowWaves)),
                   dim3(kWaveRowWaves * kWave), 0, st, w.scores, w.nsp, a.q_pos, a.m, a.n_cap, a.k, a.Tq, t0, tcur, tb,
                   nrows, a.topk_idx, a.topk_score);
      } else {
        LCS_LAUNCH("topk_rowwise_kernel", topk_rowwise_kernel, dim3((unsigned)(a.B * tcur)), dim3(kSelThreads), 0,
                   st, w.scores, w.comb, w.nsp, a.q_pos, a.m, a.n_cap, a.k, a.Tq, t0, tcur, tb, a.topk_idx,
                   a.topk_score);
      }
    }
    if (a.append && launch_decode_append(*a.append, st)) return 4;
  }
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
