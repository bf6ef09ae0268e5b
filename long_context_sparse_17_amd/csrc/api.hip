// C ABI of the hybrid compressed attention forward: argument validation, workspace queries, and
// kernel launches on the caller's stream.  Declarations and the contract are in include/lcs.h.
#include <hip/hip_runtime.h>

#include <cmath>
#include <atomic>
#include <mutex>
#include <string>
#include <utility>
#include <vector>

#include "../../include/lcs.h"
#include "common.h"
#include "kernels.h"

namespace {

constexpr int kVersion = 10000;  // 1.0.0

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool aligned4(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 3u) == 0; }

// ------------------------------------------------------------------------------ timing facility
struct Timing {
  std::mutex mu;
  std::atomic<bool> on{false};
  struct Rec { std::string name; hipEvent_t a, b; };
  std::vector<Rec> recs;
  std::vector<hipEvent_t> pool;
  hipEvent_t pending = nullptr;
  hipEvent_t get() {
    if (!pool.empty()) { hipEvent_t e = pool.back(); pool.pop_back(); return e; }
    // Timing-only events: no system-scope fence when one is recorded, so recording it neither
    // writes back nor invalidates the caches between the launches it brackets.
    hipEvent_t e = nullptr;
    if (hipEventCreateWithFlags(&e, hipEventDisableSystemFence) != hipSuccess) return nullptr;
    return e;
  }
};
Timing& timing() {
  static Timing t;
  return t;
}

}  // namespace

namespace lcs {
RopeFreq rope_freq(float theta) {
  RopeFreq f;
  for (int j = 0; j < kRopeDims / 2; ++j) f.inv[j] = std::pow((double)theta, -(double)j / (kRopeDims / 2));
  return f;
}

void timing_before(const char*, hipStream_t s) {
  Timing& t = timing();
  if (!t.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(t.mu);
  t.pending = t.get();
  if (t.pending && hipEventRecord(t.pending, s) != hipSuccess) {   // this launch goes untimed
    t.pool.push_back(t.pending);
    t.pending = nullptr;
  }
}
void timing_after(const char* name, hipStream_t s) {
  Timing& t = timing();
  if (!t.on.load(std::memory_order_relaxed)) return;
  std::lock_guard<std::mutex> lk(t.mu);
  if (!t.pending) return;
  hipEvent_t b = t.get();
  if (!b || hipEventRecord(b, s) != hipSuccess) {                  // this launch goes untimed
    if (b) t.pool.push_back(b);
    t.pool.push_back(t.pending);
    t.pending = nullptr;
    return;
  }
  t.recs.push_back({name, t.pending, b});
  t.pending = nullptr;
}
}  // namespace lcs

extern "C" {

int lcs_version(void) { return kVersion; }

const char* lcs_status_string(int status) {
  switch (status) {
    case LCS_OK: return "ok";
    case LCS_ERR_ARG: return "invalid argument";
    case LCS_ERR_UNSUPPORTED: return "unsupported shape or dtype";
    case LCS_ERR_WORKSPACE: return "workspace too small";
    case LCS_ERR_HIP: return "HIP launch error";
    case LCS_ERR_SCRATCH: return "shape needs more than the library's static scratch holds";
    default: return "unknown status";
  }
}

int lcs_timing_enable(int on) {
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  if (!on) {
    for (auto& r : t.recs) { (void)hipEventDestroy(r.a); (void)hipEventDestroy(r.b); }
    for (auto e : t.pool) (void)hipEventDestroy(e);
    t.recs.clear();
    t.pool.clear();
  }
  t.on = on != 0;
  return LCS_OK;
}

int lcs_timing_read(const char* name, double* total_ms, int64_t* launches) {
  if (!name || !total_ms || !launches) return LCS_ERR_ARG;
  Timing& t = timing();
  std::lock_guard<std::mutex> lk(t.mu);
  double tot = 0.0;
  int64_t n = 0;
  for (auto& r : t.recs) {
    if (r.name.find(name) == std::string::npos) continue;
    if (hipEventSynchronize(r.b) != hipSuccess) return LCS_ERR_HIP;
    float ms = 0.f;
    if (hipEventElapsedTime(&ms, r.a, r.b) != hipSuccess) return LCS_ERR_HIP;
    tot += ms;
    ++n;
  }
  *total_ms = tot;
  *launches = n;
  return LCS_OK;
}

// ------------------------------------------------------------------------------ compression
static int compress_common(const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok,
                           const float* ik_score, int B, int T, int64_t tok0, int64_t blk_begin, int n_blk,
                           int m, int overlap, int c, int dI, const uint16_t* gamma_kv, float eps,
                           float rope_theta, int64_t rope_offset, uint16_t* kv_out, int64_t kv_ld,
                           int64_t ring_cap, void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype,
                           void* stream) {
  if (!kv_tok || !kv_score || !gamma_kv || !kv_out) return LCS_ERR_ARG;
  if (B <= 0 || T <= 0 || n_blk <= 0 || m <= 0 || overlap < 0 || blk_begin < 0 || kv_ld <= 0 || ring_cap < 0)
    return LCS_ERR_ARG;
  if (!(eps >= 0.f) || !(rope_theta > 0.f)) return LCS_ERR_ARG;
  if (!aligned16(kv_tok) || !aligned16(kv_out) || !aligned16(gamma_kv) || !aligned4(kv_score)) return LCS_ERR_ARG;
  if (c != LCS_HEAD_DIM) return LCS_ERR_UNSUPPORTED;
  if (overlap > 4 * m || (int64_t)m + overlap > 1024) return LCS_ERR_UNSUPPORTED;
  // every pooled token of the requested blocks must be inside [tok0, tok0 + T)
  int64_t lo = blk_begin * m - overlap;
  if (lo < 0) lo = 0;
  const int64_t hi = (blk_begin + n_blk) * (int64_t)m;
  if (lo < tok0 || hi > tok0 + T) return LCS_ERR_ARG;
  const int64_t last = blk_begin + n_blk - 1;
  if (ring_cap > 0 ? ring_cap > kv_ld : last >= kv_ld) return LCS_ERR_ARG;
  if (ring_cap > 0 && n_blk > ring_cap) return LCS_ERR_ARG;  // two entries of one call would share a row
  const bool has_ik = ik_tok != nullptr;
  if (has_ik) {
    if (!ik_score || !ik_out || ik_ld <= 0) return LCS_ERR_ARG;
    if (ik_dtype != LCS_IK_BF16 && ik_dtype != LCS_IK_FP8) return LCS_ERR_UNSUPPORTED;
    if (dI != 64 && dI != 128) return LCS_ERR_UNSUPPORTED;
    if (ik_dtype == LCS_IK_FP8 && !ik_scale) return LCS_ERR_ARG;
    if (last >= ik_ld) return LCS_ERR_ARG;
  }
  lcs::CompressArgs a;
  a.kv_tok = kv_tok; a.kv_score = kv_score; a.ik_tok = has_ik ? ik_tok : nullptr; a.ik_score = ik_score;
  a.B = B; a.T = T; a.tok0 = tok0; a.blk_begin = blk_begin; a.n_blk = n_blk; a.m = m; a.ov = overlap;
  a.dI = has_ik ? dI : 0; a.gamma = gamma_kv; a.eps = eps; a.theta = rope_theta; a.rope_offset = rope_offset;
  a.kv_out = kv_out; a.kv_ld = kv_ld; a.ring_cap = ring_cap; a.ik_out = ik_out; a.ik_scale = ik_scale;
  a.ik_ld = ik_ld; a.ik_fp8 = ik_dtype == LCS_IK_FP8;
  if (B > 65535) return LCS_ERR_UNSUPPORTED;
  return lcs::launch_compress(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

int csa_compress_kv(const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok, const float* ik_score,
                    int B, int T, int64_t tok0, int64_t blk_begin, int n_blk, int m, int overlap, int c, int dI,
                    const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset, uint16_t* kv_out,
                    int64_t kv_ld, int64_t ring_cap, void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype,
                    void* stream) {
  return compress_common(kv_tok, kv_score, ik_tok, ik_score, B, T, tok0, blk_begin, n_blk, m, overlap, c, dI,
                         gamma_kv, eps, rope_theta, rope_offset, kv_out, kv_ld, ring_cap, ik_out, ik_scale, ik_ld,
                         ik_dtype, stream);
}

int hca_compress_kv(const uint16_t* kv_tok, const float* kv_score, int B, int T, int64_t tok0, int64_t blk_begin,
                    int n_blk, int m, int c, const uint16_t* gamma_kv, float eps, float rope_theta,
                    int64_t rope_offset, uint16_t* kv_out, int64_t kv_ld, int64_t ring_cap, void* stream) {
  return compress_common(kv_tok, kv_score, nullptr, nullptr, B, T, tok0, blk_begin, n_blk, m, 0, c, 0, gamma_kv,
                         eps, rope_theta, rope_offset, kv_out, kv_ld, ring_cap, nullptr, nullptr, 0, 0, stream);
}

// ------------------------------------------------------------------------------ decode append
size_t kv_decode_state_bytes(int B) { return B > 0 ? lcs::decode_state_bytes(B) : 0; }

}  // extern "C"

// Checks of kv_decode_append's arguments; fills the launch arguments when they pass.
static int append_args(const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok, const float* ik_score,
                       const int64_t* pos, int B, int m, int overlap, int c, int dI, const uint16_t* gamma_kv,
                       float eps, float rope_theta, int64_t rope_offset, float* state, size_t state_bytes,
                       int kv_dtype, void* win, float* win_scale, int64_t win_ld, int64_t ring_cap, void* kv_out,
                       float* kv_scale, int64_t kv_ld, int64_t kv_ring, void* ik_out, float* ik_scale, int64_t ik_ld,
                       int ik_dtype, lcs::DecodeAppendArgs* out) {
  if (!kv_tok || !kv_score || !pos || !gamma_kv || !state || !kv_out) return LCS_ERR_ARG;
  if (B <= 0 || m <= 0 || overlap < 0 || kv_ld <= 0 || kv_ring < 0) return LCS_ERR_ARG;
  if (!(eps >= 0.f) || !(rope_theta > 0.f)) return LCS_ERR_ARG;
  if (!aligned16(kv_tok) || !aligned16(kv_out) || !aligned16(gamma_kv) || !aligned16(state) || !aligned4(kv_score) ||
      (reinterpret_cast<uintptr_t>(pos) & 7u))
    return LCS_ERR_ARG;
  if (c != LCS_HEAD_DIM) return LCS_ERR_UNSUPPORTED;
  if (overlap > m) return LCS_ERR_UNSUPPORTED;                 // a token lies in at most two blocks
  if (state_bytes < lcs::decode_state_bytes(B)) return LCS_ERR_WORKSPACE;
  if (kv_dtype != LCS_KV_BF16 && kv_dtype != LCS_KV_FP8) return LCS_ERR_UNSUPPORTED;
  const bool kv8 = kv_dtype == LCS_KV_FP8;
  if (kv8 && (!kv_scale || !aligned4(kv_scale) || (win && (!win_scale || !aligned4(win_scale))))) return LCS_ERR_ARG;
  if (kv_ring > kv_ld) return LCS_ERR_ARG;
  if (win && (ring_cap <= 0 || win_ld < ring_cap || !aligned16(win))) return LCS_ERR_ARG;
  const bool has_ik = ik_tok != nullptr;
  if (has_ik) {
    if (!ik_score || !ik_out || ik_ld <= 0) return LCS_ERR_ARG;
    if (ik_dtype != LCS_IK_BF16 && ik_dtype != LCS_IK_FP8) return LCS_ERR_UNSUPPORTED;
    if (dI != 64 && dI != 128) return LCS_ERR_UNSUPPORTED;
    if (ik_dtype == LCS_IK_FP8 && !ik_scale) return LCS_ERR_ARG;
  }
  lcs::DecodeAppendArgs& a = *out;
  a.kv_tok = kv_tok; a.kv_score = kv_score; a.ik_tok = has_ik ? ik_tok : nullptr; a.ik_score = ik_score;
  a.pos = pos; a.B = B; a.m = m; a.ov = overlap; a.dI = has_ik ? dI : 0;
  a.gamma = gamma_kv; a.eps = eps; a.theta = rope_theta; a.rope_offset = rope_offset;
  a.state = state; a.win = win; a.win_ld = win_ld; a.ring_cap = ring_cap;
  a.kv_out = kv_out; a.kv_ld = kv_ld; a.kv_ring = kv_ring;
  a.kv8 = kv8; a.win_scale = win_scale; a.kv_scale = kv_scale;
  a.ik_out = ik_out; a.ik_scale = ik_scale; a.ik_ld = ik_ld; a.ik_fp8 = ik_dtype == LCS_IK_FP8;
  return LCS_OK;
}

extern "C" {

int kv_decode_append(const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok, const float* ik_score,
                     const int64_t* pos, int B, int m, int overlap, int c, int dI, const uint16_t* gamma_kv,
                     float eps, float rope_theta, int64_t rope_offset, float* state, size_t state_bytes,
                     int kv_dtype, void* win, float* win_scale, int64_t win_ld, int64_t ring_cap, void* kv_out,
                     float* kv_scale, int64_t kv_ld, int64_t kv_ring, void* ik_out, float* ik_scale, int64_t ik_ld,
                     int ik_dtype, void* stream) {
  lcs::DecodeAppendArgs a;
  const int st = append_args(kv_tok, kv_score, ik_tok, ik_score, pos, B, m, overlap, c, dI, gamma_kv, eps, rope_theta,
                             rope_offset, state, state_bytes, kv_dtype, win, win_scale, win_ld, ring_cap, kv_out,
                             kv_scale, kv_ld, kv_ring, ik_out, ik_scale, ik_ld, ik_dtype, &a);
  if (st != LCS_OK) return st;
  return lcs::launch_decode_append(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

// ------------------------------------------------------------------------------ input projections
int input_proj(const uint16_t* h, int M, int d, const uint16_t* w_in, int n_rows, int n_seg, const int* seg_width,
               void* const* seg_dst, const int64_t* seg_ld, const int* seg_fp32, void* stream) {
  if (!h || !w_in || !seg_width || !seg_dst || !seg_ld || !seg_fp32) return LCS_ERR_ARG;
  if (M <= 0 || d <= 0 || n_rows <= 0 || n_seg <= 0) return LCS_ERR_ARG;
  if (!aligned16(h) || !aligned16(w_in)) return LCS_ERR_ARG;
  if (M > 8 || (d != 4096 && d != 8192) || n_rows % 16 != 0 || n_seg > lcs::kMaxProjSegments)
    return LCS_ERR_UNSUPPORTED;
  lcs::ProjSegments seg{};
  seg.n = n_seg;
  int64_t end = 0;
  for (int i = 0; i < n_seg; ++i) {
    if (seg_width[i] <= 0 || !seg_dst[i] || seg_ld[i] < seg_width[i]) return LCS_ERR_ARG;
    if (seg_fp32[i] ? !aligned4(seg_dst[i]) : (reinterpret_cast<uintptr_t>(seg_dst[i]) & 1u)) return LCS_ERR_ARG;
    end += seg_width[i];
    if (end > n_rows) return LCS_ERR_ARG;
    seg.end[i] = (int)end; seg.dst[i] = seg_dst[i]; seg.ld[i] = seg_ld[i]; seg.f32[i] = seg_fp32[i] != 0;
  }
  return lcs::launch_input_proj(h, M, d, w_in, n_rows, seg, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

// ------------------------------------------------------------------------------ fp8 K=V rows
int kv_quantize_fp8(const uint16_t* kv, int64_t rows, uint8_t* codes, float* scales, void* stream) {
  if (!kv || !codes || !scales || rows <= 0) return LCS_ERR_ARG;
  if (!aligned16(kv) || !aligned16(codes) || !aligned4(scales)) return LCS_ERR_ARG;
  if (rows > ((int64_t)1 << 33)) return LCS_ERR_UNSUPPORTED;
  return lcs::launch_kv_quantize(kv, rows, codes, scales, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

// ------------------------------------------------------------------------------ mHC
int mhc_sinkhorn(const float* logits, int T, int n, int iters, float* b_out, void* stream) {
  if (!logits || !b_out || T <= 0 || iters < 1 || iters > 10000) return LCS_ERR_ARG;
  if (!aligned4(logits) || !aligned4(b_out)) return LCS_ERR_ARG;
  if (n < 1 || n > 8) return LCS_ERR_UNSUPPORTED;
  lcs::MhcArgs a{};
  a.logits = logits; a.T = T; a.n = n; a.iters = iters; a.b_out = b_out;
  return lcs::launch_mhc(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

int mhc_mix(const uint16_t* x, const uint16_t* y, const float* logits, int T, int n, int d, int iters,
            uint16_t* x_out, uint16_t* h_out, void* stream) {
  if (!x || !y || !logits || !x_out || T <= 0 || d <= 0 || iters < 1 || iters > 10000) return LCS_ERR_ARG;
  if (!aligned16(x) || !aligned16(y) || !aligned16(x_out) || (h_out && !aligned16(h_out)) || !aligned4(logits))
    return LCS_ERR_ARG;
  if (n < 1 || n > 8 || d % 8 != 0) return LCS_ERR_UNSUPPORTED;
  lcs::MhcArgs a{};
  a.x = x; a.y = y; a.logits = logits; a.T = T; a.n = n; a.d = d; a.iters = iters; a.x_out = x_out; a.h_out = h_out;
  return lcs::launch_mhc(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

// ------------------------------------------------------------------------------ indexer + top-k
size_t csa_index_topk_state_bytes(void) { return lcs::index_topk_state_bytes(); }

size_t csa_index_topk_workspace(int B, int Tq, int64_t n_cap, int k) {
  if (B <= 0 || Tq <= 0 || n_cap <= 0 || k <= 0) return 0;
  return lcs::index_topk_workspace(B, Tq, n_cap, k);
}

}  // extern "C"

// Checks of csa_index_topk's arguments; fills the launch arguments when they pass.
static int index_args(const uint16_t* q_idx, const uint16_t* w_idx, const void* ik_cache, const float* ik_scale,
                      int64_t ik_ld, int ik_dtype, const int64_t* q_pos, int64_t n_cap, int B, int Tq, int H_I,
                      int dI, int m, int k, int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                      lcs::IndexArgs* out) {
  if (!q_idx || !w_idx || !ik_cache || !q_pos || !topk_idx) return LCS_ERR_ARG;
  if (B <= 0 || Tq <= 0 || H_I <= 0 || m <= 0 || k <= 0 || n_cap <= 0 || ik_ld < n_cap) return LCS_ERR_ARG;
  if (!aligned16(q_idx) || !aligned16(ik_cache) || !aligned4(topk_idx)) return LCS_ERR_ARG;
  if (ik_dtype != LCS_IK_BF16 && ik_dtype != LCS_IK_FP8) return LCS_ERR_UNSUPPORTED;
  if (ik_dtype == LCS_IK_FP8 && (!ik_scale || dI != 128)) return ik_scale ? LCS_ERR_UNSUPPORTED : LCS_ERR_ARG;
  if (dI != 64 && dI != 128) return LCS_ERR_UNSUPPORTED;
  if (H_I > LCS_MAX_HEADS || k > LCS_MAX_TOPK) return LCS_ERR_UNSUPPORTED;
  if (n_cap >= ((int64_t)1 << 31)) return LCS_ERR_UNSUPPORTED;
  if ((int64_t)B * Tq > 65535 * 16) return LCS_ERR_UNSUPPORTED;
  if (!lcs::index_topk_launchable(B, Tq, n_cap, ik_dtype == LCS_IK_FP8)) return LCS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < lcs::index_topk_workspace(B, Tq, n_cap, k)) return LCS_ERR_WORKSPACE;
  if (!aligned16(ws)) return LCS_ERR_ARG;
  lcs::IndexArgs& a = *out;
  a.q_idx = q_idx; a.w_idx = w_idx; a.ik = ik_cache; a.ik_scale = ik_scale; a.ik_ld = ik_ld;
  a.ik_fp8 = ik_dtype == LCS_IK_FP8; a.q_pos = q_pos; a.n_cap = n_cap; a.B = B; a.Tq = Tq; a.H_I = H_I;
  a.dI = dI; a.m = m; a.k = k; a.topk_idx = topk_idx; a.topk_score = topk_score; a.ws = ws; a.ws_bytes = ws_bytes;
  a.append = nullptr;
  return LCS_OK;
}

extern "C" {

int csa_index_topk(const uint16_t* q_idx, const uint16_t* w_idx, const void* ik_cache, const float* ik_scale,
                   int64_t ik_ld, int ik_dtype, const int64_t* q_pos, int64_t n_cap, int B, int Tq, int H_I,
                   int dI, int m, int k, int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                   void* stream) {
  lcs::IndexArgs a;
  const int st = index_args(q_idx, w_idx, ik_cache, ik_scale, ik_ld, ik_dtype, q_pos, n_cap, B, Tq, H_I, dI, m, k,
                            topk_idx, topk_score, ws, ws_bytes, &a);
  if (st != LCS_OK) return st;
  return lcs::launch_index_topk(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

int csa_index_topk_append(const uint16_t* q_idx, const uint16_t* w_idx, const void* ik_cache, const float* ik_scale,
                          int64_t ik_ld, int ik_dtype, const int64_t* q_pos, int64_t n_cap, int B, int Tq, int H_I,
                          int dI, int m, int k, int32_t* topk_idx, float* topk_score, void* ws, size_t ws_bytes,
                          const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok,
                          const float* ik_score, const int64_t* pos, int B_app, int m_app, int overlap, int c,
                          int dI_app, const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset,
                          float* state, size_t state_bytes, int kv_dtype, void* win, float* win_scale,
                          int64_t win_ld, int64_t ring_cap, void* kv_out, float* kv_scale, int64_t kv_ld,
                          int64_t kv_ring, void* ik_out, float* ik_out_scale, int64_t ik_out_ld, int ik_out_dtype,
                          void* stream) {
  lcs::IndexArgs a;
  int st = index_args(q_idx, w_idx, ik_cache, ik_scale, ik_ld, ik_dtype, q_pos, n_cap, B, Tq, H_I, dI, m, k, topk_idx,
                      topk_score, ws, ws_bytes, &a);
  if (st != LCS_OK) return st;
  lcs::DecodeAppendArgs ap;
  st = append_args(kv_tok, kv_score, ik_tok, ik_score, pos, B_app, m_app, overlap, c, dI_app, gamma_kv, eps,
                   rope_theta, rope_offset, state, state_bytes, kv_dtype, win, win_scale, win_ld, ring_cap, kv_out,
                   kv_scale, kv_ld, kv_ring, ik_out, ik_out_scale, ik_out_ld, ik_out_dtype, &ap);
  if (st != LCS_OK) return st;
  a.append = &ap;
  return lcs::launch_index_topk(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

// ------------------------------------------------------------------------------ attention
size_t lcs_attend_workspace(int B, int Tq, int H, int64_t max_keys) {
  if (B <= 0 || Tq <= 0 || H <= 0 || max_keys < 0) return 0;
  return lcs::attend_workspace(B, Tq, H, max_keys);
}

static int attend_common(const uint16_t* q, const uint16_t* gamma_q, const uint16_t* kv_cache, int64_t kv_ld,
                         const int32_t* topk_idx, int k, int64_t n_cap, int m, const uint16_t* win_ring,
                         int64_t win_ld, int64_t ring_cap, int window, const float* sink, const int64_t* q_pos,
                         int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
                         uint16_t* out, void* ws, size_t ws_bytes, void* stream, int64_t max_keys,
                         const float* kv_scale = nullptr, const float* win_scale = nullptr, bool kv8 = false,
                         const lcs::DecodeAppendArgs* append = nullptr) {
  if (!q || !gamma_q || !kv_cache || !sink || !q_pos || !out) return LCS_ERR_ARG;
  if (kv8 && (!kv_scale || !aligned4(kv_scale) || (window > 0 && (!win_scale || !aligned4(win_scale)))))
    return LCS_ERR_ARG;
  if (window > 0 && !win_ring) return LCS_ERR_ARG;
  if (B <= 0 || Tq <= 0 || H <= 0 || kv_ld <= 0 || window < 0 || ring_cap < 0) return LCS_ERR_ARG;
  if (window > 0 && win_ld <= 0) return LCS_ERR_ARG;
  if (ring_cap > 0 && (ring_cap > win_ld || ring_cap < window)) return LCS_ERR_ARG;
  if (!aligned16(q) || !aligned16(gamma_q) || !aligned16(kv_cache) || !aligned16(out)) return LCS_ERR_ARG;
  if (win_ring && !aligned16(win_ring)) return LCS_ERR_ARG;
  if (!(scale > 0.f) || !(eps >= 0.f) || !(rope_theta > 0.f)) return LCS_ERR_ARG;
  if (c != LCS_HEAD_DIM || H > LCS_MAX_HEADS) return LCS_ERR_UNSUPPORTED;
  if ((int64_t)B * Tq > 65535) return LCS_ERR_UNSUPPORTED;
  if (max_keys >= ((int64_t)1 << 31)) return LCS_ERR_UNSUPPORTED;
  if (!lcs::attend_launchable(B, Tq, H, max_keys, topk_idx != nullptr)) return LCS_ERR_UNSUPPORTED;
  if (!ws || ws_bytes < lcs::attend_workspace(B, Tq, H, max_keys)) return LCS_ERR_WORKSPACE;
  if (!aligned16(ws)) return LCS_ERR_ARG;
  lcs::AttendArgs a;
  a.q = q; a.gamma_q = gamma_q; a.kv = kv8 ? nullptr : kv_cache; a.kv_ld = kv_ld; a.topk = topk_idx; a.k = k;
  a.n_cap = n_cap;
  a.kv8 = kv8 ? reinterpret_cast<const uint8_t*>(kv_cache) : nullptr; a.kv_scale = kv_scale;
  a.win8 = kv8 ? reinterpret_cast<const uint8_t*>(win_ring) : nullptr; a.win_scale = win_scale;
  a.m = m; a.win = kv8 ? nullptr : win_ring; a.win_ld = win_ld; a.ring_cap = ring_cap; a.window = window; a.sink = sink;
  a.q_pos = q_pos; a.rope_offset = rope_offset; a.B = B; a.Tq = Tq; a.H = H; a.scale = scale; a.eps = eps;
  a.theta = rope_theta; a.out = out; a.ws = ws; a.ws_bytes = ws_bytes;
  a.append = append;
  if (!win_ring) {
    // no window ring (window = 0): the kernels still form addresses for padding slots of a tile, so
    // point the ring at the cache itself (same row layout, never scored)
    if (kv8) { a.win8 = a.kv8; a.win_scale = kv_scale; }
    else a.win = kv_cache;
    a.win_ld = kv_ld;
    a.ring_cap = 0;
  }
  return lcs::launch_attend(a, max_keys, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

int csa_attend(const uint16_t* q, const uint16_t* gamma_q, const uint16_t* kv_cache, int64_t kv_ld,
               const int32_t* topk_idx, int k, const uint16_t* win_ring, int64_t win_ld, int64_t ring_cap,
               int window, const float* sink, const int64_t* q_pos, int64_t rope_offset, int B, int Tq, int H,
               int c, float scale, float eps, float rope_theta, uint16_t* out, void* ws, size_t ws_bytes,
               void* stream) {
  if (!topk_idx || k <= 0) return LCS_ERR_ARG;
  if (!aligned4(topk_idx)) return LCS_ERR_ARG;
  if (k > LCS_MAX_TOPK) return LCS_ERR_UNSUPPORTED;
  return attend_common(q, gamma_q, kv_cache, kv_ld, topk_idx, k, 0, 1, win_ring, win_ld, ring_cap, window, sink,
                       q_pos, rope_offset, B, Tq, H, c, scale, eps, rope_theta, out, ws, ws_bytes, stream,
                       (int64_t)k + window);
}

int hca_attend(const uint16_t* q, const uint16_t* gamma_q, const uint16_t* kv_cache, int64_t kv_ld, int64_t n_cap,
               int m, const uint16_t* win_ring, int64_t win_ld, int64_t ring_cap, int window, const float* sink,
               const int64_t* q_pos, int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps,
               float rope_theta, uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (m <= 0 || n_cap < 0 || n_cap > kv_ld) return LCS_ERR_ARG;
  return attend_common(q, gamma_q, kv_cache, kv_ld, nullptr, 0, n_cap, m, win_ring, win_ld, ring_cap, window,
                       sink, q_pos, rope_offset, B, Tq, H, c, scale, eps, rope_theta, out, ws, ws_bytes, stream,
                       n_cap + window);
}

int csa_attend_kv8(const uint16_t* q, const uint16_t* gamma_q, const uint8_t* kv_codes, const float* kv_scale,
                   int64_t kv_ld, const int32_t* topk_idx, int k, const uint8_t* win_codes, const float* win_scale,
                   int64_t win_ld, int64_t ring_cap, int window, const float* sink, const int64_t* q_pos,
                   int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
                   uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (!topk_idx || k <= 0) return LCS_ERR_ARG;
  if (!aligned4(topk_idx)) return LCS_ERR_ARG;
  if (k > LCS_MAX_TOPK) return LCS_ERR_UNSUPPORTED;
  return attend_common(q, gamma_q, reinterpret_cast<const uint16_t*>(kv_codes), kv_ld, topk_idx, k, 0, 1,
                       reinterpret_cast<const uint16_t*>(win_codes), win_ld, ring_cap, window, sink, q_pos,
                       rope_offset, B, Tq, H, c, scale, eps, rope_theta, out, ws, ws_bytes, stream,
                       (int64_t)k + window, kv_scale, win_scale, true);
}

int hca_attend_kv8(const uint16_t* q, const uint16_t* gamma_q, const uint8_t* kv_codes, const float* kv_scale,
                   int64_t kv_ld, int64_t n_cap, int m, const uint8_t* win_codes, const float* win_scale,
                   int64_t win_ld, int64_t ring_cap, int window, const float* sink, const int64_t* q_pos,
                   int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
                   uint16_t* out, void* ws, size_t ws_bytes, void* stream) {
  if (m <= 0 || n_cap < 0 || n_cap > kv_ld) return LCS_ERR_ARG;
  return attend_common(q, gamma_q, reinterpret_cast<const uint16_t*>(kv_codes), kv_ld, nullptr, 0, n_cap, m,
                       reinterpret_cast<const uint16_t*>(win_codes), win_ld, ring_cap, window, sink, q_pos,
                       rope_offset, B, Tq, H, c, scale, eps, rope_theta, out, ws, ws_bytes, stream, n_cap + window,
                       kv_scale, win_scale, true);
}

int hca_attend_append(const uint16_t* q, const uint16_t* gamma_q, int64_t n_cap, int window, const float* sink,
                      const int64_t* q_pos, int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps,
                      float rope_theta, uint16_t* out, void* ws, size_t ws_bytes, const uint16_t* kv_tok,
                      const float* kv_score, const uint16_t* ik_tok, const float* ik_score, const int64_t* pos,
                      int B_app, int m, int overlap, int c_app, int dI, const uint16_t* gamma_kv, float eps_kv,
                      float rope_theta_kv, int64_t rope_offset_kv, float* state, size_t state_bytes, int kv_dtype,
                      void* win, float* win_scale, int64_t win_ld, int64_t ring_cap, void* kv_out, float* kv_scale,
                      int64_t kv_ld, int64_t kv_ring, void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype,
                      void* stream) {
  lcs::DecodeAppendArgs ap;
  const int st = append_args(kv_tok, kv_score, ik_tok, ik_score, pos, B_app, m, overlap, c_app, dI, gamma_kv, eps_kv,
                             rope_theta_kv, rope_offset_kv, state, state_bytes, kv_dtype, win, win_scale, win_ld,
                             ring_cap, kv_out, kv_scale, kv_ld, kv_ring, ik_out, ik_scale, ik_ld, ik_dtype, &ap);
  if (st != LCS_OK) return st;
  // one query per sequence, the append's batch; the attention reads the stores the append writes
  if (Tq != 1 || B_app != B || kv_ring != 0) return LCS_ERR_UNSUPPORTED;
  if (n_cap < 0 || n_cap > kv_ld) return LCS_ERR_ARG;
  if (window > 0 && !win) return LCS_ERR_ARG;
  const bool kv8 = kv_dtype == LCS_KV_FP8;
  return attend_common(q, gamma_q, static_cast<const uint16_t*>(kv_out), kv_ld, nullptr, 0, n_cap, m,
                       static_cast<const uint16_t*>(win), win_ld, ring_cap, window, sink, q_pos, rope_offset, B, Tq,
                       H, c, scale, eps, rope_theta, out, ws, ws_bytes, stream, n_cap + window, kv_scale, win_scale,
                       kv8, &ap);
}

// ------------------------------------------------------------------------------ grouped projection
size_t grouped_out_proj_workspace(int M, int g, int d_g) {
  if (M <= 0 || g <= 0 || d_g <= 0) return 0;
  return lcs::out_proj_workspace(M, g, d_g);
}

// Shape, pointer and alignment checks shared by the grouped-projection entry points.
static int out_proj_check(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, int M, int H, int c, int g,
                          int d_g, int d, const uint16_t* resid, const uint16_t* y) {
  if (!o || !w_g || !w_o || !y) return LCS_ERR_ARG;
  if (resid && !aligned16(resid)) return LCS_ERR_ARG;
  if (M <= 0 || H <= 0 || c <= 0 || g <= 0 || d_g <= 0 || d <= 0) return LCS_ERR_ARG;
  if (!aligned16(o) || !aligned16(w_g) || !aligned16(w_o) || !aligned16(y)) return LCS_ERR_ARG;
  if (H % g != 0 || d_g % 16 != 0 || d % 16 != 0 || ((int64_t)H / g * c) % 32 != 0 || ((int64_t)g * d_g) % 32 != 0)
    return LCS_ERR_UNSUPPORTED;
  if ((int64_t)g * d_g / 16 > 65535 * 16 || d / 16 > 65535 * 16) return LCS_ERR_UNSUPPORTED;
  return LCS_OK;
}

static int out_proj_common(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, int M, int H, int c, int g,
                           int d_g, int d, const uint16_t* resid, uint16_t* y, void* ws, size_t ws_bytes,
                           void* stream) {
  const int chk = out_proj_check(o, w_g, w_o, M, H, c, g, d_g, d, resid, y);
  if (chk != LCS_OK) return chk;
  if (!ws || ws_bytes < lcs::out_proj_workspace(M, g, d_g)) return LCS_ERR_WORKSPACE;
  if (!aligned16(ws)) return LCS_ERR_ARG;
  lcs::OutProjArgs a;
  a.o = o; a.w_g = w_g; a.w_o = w_o; a.M = M; a.H = H; a.c = c; a.g = g; a.d_g = d_g; a.d = d; a.y = y; a.ws = ws;
  a.ws_bytes = ws_bytes; a.resid = resid;
  return lcs::launch_out_proj(a, static_cast<hipStream_t>(stream)) ? LCS_ERR_HIP : LCS_OK;
}

int grouped_out_proj(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, int M, int H, int c, int g,
                     int d_g, int d, uint16_t* y, void* ws, size_t ws_bytes, void* stream) {
  return out_proj_common(o, w_g, w_o, M, H, c, g, d_g, d, nullptr, y, ws, ws_bytes, stream);
}

int grouped_out_proj_residual(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, const uint16_t* resid,
                              int M, int H, int c, int g, int d_g, int d, uint16_t* y, void* ws, size_t ws_bytes,
                              void* stream) {
  if (!resid) return LCS_ERR_ARG;
  return out_proj_common(o, w_g, w_o, M, H, c, g, d_g, d, resid, y, ws, ws_bytes, stream);
}

size_t grouped_out_proj_noalloc_max_bytes(void) { return lcs::kOutProjScratchBytes; }

int grouped_out_proj_noalloc(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, int M, int H, int c,
                             int g, int d_g, int d, uint16_t* y, void* stream) {
  // every argument check before any HIP call: a rejected call touches no device
  const int chk = out_proj_check(o, w_g, w_o, M, H, c, g, d_g, d, nullptr, y);
  if (chk != LCS_OK) return chk;
  if (lcs::out_proj_workspace(M, g, d_g) > lcs::kOutProjScratchBytes) return LCS_ERR_SCRATCH;
  void* z = nullptr;
  if (lcs::out_proj_scratch(&z) != 0) return LCS_ERR_HIP;
  return out_proj_common(o, w_g, w_o, M, H, c, g, d_g, d, nullptr, y, z, lcs::kOutProjScratchBytes, stream);
}

}  // extern "C"
