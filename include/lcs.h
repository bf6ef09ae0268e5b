/*
 * lcs.h -- C ABI of the MI355X (gfx950) hybrid compressed attention forward (CSA + HCA).
 *
 * The method is the DeepSeek-V4 attention described on page 1 ("DeepSeek V4 ..." walk-through,
 * section "hybrid attention", CSA steps 1-4, the HCA paragraph, Q/KV normalization, partial RoPE,
 * the sliding-window branch and the attention sink) and page 4 ("DeepSeek-V4开源解读",
 * section 3.1 "Hybrid Attention: CSA + HCA", the Flash constants).
 *
 * Conventions for every entry point:
 *   - Data pointers are DEVICE pointers owned by the caller.  The library allocates nothing on the
 *     device and keeps no state between calls, with two exceptions: grouped_out_proj_noalloc's
 *     static scratch array and the optional timing facility at the end.
 *   - Work is enqueued on `stream` (a hipStream_t; NULL = the null stream) and runs asynchronously;
 *     faults during execution surface at the caller's next synchronisation.
 *   - bf16 = uint16_t bit pattern; fp8 = uint8_t OCP E4M3FN; positions are int64 token indices.
 *   - Tensors are row-major and contiguous, shapes given in [] with the fastest axis last.
 *     Caches carry an explicit per-sequence row count ("ld"): row r of sequence b starts at
 *     element (b*ld + r) * width.
 *   - Return value: LCS_OK, or an error code below; on error nothing has been enqueued.
 *   - Device-side preconditions that would need a synchronisation to check are documented, not
 *     checked: finite inputs, indices in range, positions inside the buffers.
 *   - Same inputs give bitwise-identical outputs (no floating-point atomics anywhere).
 *
 * Readings of the pages that fix the arithmetic (page 1, section "hybrid attention", unless noted):
 *   pooling  entry i = sum_j softmax(s[S_i])_j x_j over tokens S_i = [i*m - ov, (i+1)*m), j >= 0
 *   norm     RMSNorm(x) = gamma * x / sqrt(mean(x^2) + eps) on pooled entries, window tokens, q heads
 *   rope     dims 448..511 as adjacent pairs (448+2j, 449+2j), angle = pos * theta^(-j/32);
 *            entry i at pos (i+1)*m - 1 + rope_offset, window token j at j + rope_offset, query t at
 *            t + rope_offset; the output's last 64 dims are rotated by -(t + rope_offset)
 *   visible  entry i is visible to the query at token t iff (i+1)*m <= t  (n_vis = t / m)
 *   window   tokens [max(0, t-window+1), t]; one joint softmax over compressed keys + window + sink
 *   sink     p = e^l / (e^z_h + sum e^l), l = scale * qhat . k (scale normally 1/sqrt(512))
 *   indexer  I_s = sum_h w_h * max(0, q_h . k_s)   (page 1 CSA step 2; page 4 section 3.1)
 */
#ifndef LCS_H_
#define LCS_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define LCS_OK 0
#define LCS_ERR_ARG 1          /* NULL pointer, non-positive size, bad stride or misalignment  */
#define LCS_ERR_UNSUPPORTED 2  /* shape or dtype the library does not implement                */
#define LCS_ERR_WORKSPACE 3    /* workspace NULL or smaller than the *_workspace() query      */
#define LCS_ERR_HIP 4          /* a HIP launch error                                          */
#define LCS_ERR_SCRATCH 5      /* the shape needs more than an allocation-free call's scratch */

#define LCS_IK_BF16 0          /* indexer keys stored as bf16, no scale                        */
#define LCS_IK_FP8 1           /* indexer keys stored as E4M3FN codes + one fp32 scale per key */
#define LCS_KV_BF16 0          /* K=V rows (entries, window ring) stored as bf16               */
#define LCS_KV_FP8 1           /* K=V rows stored as E4M3FN codes + one fp32 scale per row     */

#define LCS_HEAD_DIM 512       /* c, fixed (page 1, "hybrid attention", CSA step 4)           */
#define LCS_MAX_HEADS 64
#define LCS_MAX_TOPK 2048

int lcs_version(void);
const char* lcs_status_string(int status);

/*
 * csa_compress_kv -- CSA step 1 (page 1, "hybrid attention", CSA step 1; page 4 section 3.1, m = 4):
 * pools m-token blocks with an overlap of `overlap` earlier tokens into one K=V entry each, then
 * RMSNorm(gamma_kv) and RoPE at the block's last token.  With ik_tok != NULL the indexer key of the
 * block is pooled the same way with its own logits ik_score (no norm, no RoPE) and stored as bf16
 * (ik_dtype = LCS_IK_BF16) or as E4M3FN codes with scale = absmax/448 (LCS_IK_FP8).
 *
 *   kv_tok   [B, T, c] bf16   raw per-token K=V vectors of tokens tok0 .. tok0+T-1
 *   kv_score [B, T]    fp32   one pooling logit per token
 *   ik_tok   [B, T, dI] bf16, ik_score [B, T] fp32   (both NULL: no indexer keys)
 *   blocks blk_begin .. blk_begin+n_blk-1 are produced; every token they pool must lie in
 *   [tok0, tok0+T) (tokens < 0 are dropped), else LCS_ERR_ARG.
 *   kv_out   [B, kv_ld, c] bf16: entry i goes to row i (ring_cap = 0) or row i % ring_cap; with a
 *            ring, one call writes at most ring_cap entries (else LCS_ERR_ARG).
 *   ik_out   [B, ik_ld, dI] (uint8 codes or bf16), ik_scale [B, ik_ld] fp32 (fp8 only), row i.
 *   Requirements: c = 512, m >= 1, 0 <= overlap <= 4*m, m + overlap <= 1024, dI in {64, 128}.
 */
int csa_compress_kv(const uint16_t* kv_tok, const float* kv_score,
                    const uint16_t* ik_tok, const float* ik_score,
                    int B, int T, int64_t tok0, int64_t blk_begin, int n_blk,
                    int m, int overlap, int c, int dI,
                    const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset,
                    uint16_t* kv_out, int64_t kv_ld, int64_t ring_cap,
                    void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype,
                    void* stream);

/*
 * hca_compress_kv -- HCA compression (page 1, HCA paragraph: m' = 128, no overlap) and, with m = 1,
 * the sliding-window fill (page 1, "sliding window": uncompressed tokens, each normed and rotated
 * to its own position).  Same arguments and layout as csa_compress_kv without indexer keys.
 */
int hca_compress_kv(const uint16_t* kv_tok, const float* kv_score,
                    int B, int T, int64_t tok0, int64_t blk_begin, int n_blk, int m, int c,
                    const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset,
                    uint16_t* kv_out, int64_t kv_ld, int64_t ring_cap, void* stream);

/*
 * kv_decode_append -- one decode step of the compressed-KV state for B sequences, each at its own
 * position (page 1, "hybrid attention": CSA step 1, the HCA paragraph and the sliding-window branch:
 * entries pooled from m-token blocks with `overlap` earlier tokens, the nearest tokens kept
 * uncompressed).  For every b with pos[b] >= 0 the token t = pos[b] is appended:
 *   - win row t % ring_cap <- RoPE_t(RMSNorm(kv_tok[b]) * gamma_kv)        (win NULL: skipped);
 *   - the token joins the pooling state of every block containing it (block t / m and, when
 *     t >= (t/m + 1) m - overlap, the next one): online softmax over the blocks' logits, fp32;
 *   - when t = (i+1) m - 1, block i is complete: its entry (the softmax-pooled vector, RMSNorm'd,
 *     rotated to t) goes to kv_out row i (kv_ring = 0) or i % kv_ring, and its indexer key
 *     (pooled with ik_score, no norm, no RoPE) to ik_out row i as bf16 or E4M3FN + scale.
 * The result equals what csa_compress_kv / hca_compress_kv produce for the same blocks (up to the
 * order of fp32 rounding).  pos[b] < 0 leaves sequence b untouched (ragged batches).
 *
 *   kv_tok [B, c] bf16, kv_score [B] fp32, ik_tok [B, dI] bf16, ik_score [B] fp32 (NULL: no keys)
 *   pos    [B] int64 (device)
 *   state  caller-owned device buffer of >= kv_decode_state_bytes(B) bytes (16-byte aligned), kept
 *          between calls: per sequence two slots, each tagged with the block it holds.  The first
 *          token of a block (max(0, j m - overlap)) starts that block's slot; a block whose first
 *          token was never appended is not pooled and its entry is not written.  So a sequence
 *          appended from t = 0 needs no clearing; a sequence resumed mid-stream (its older blocks
 *          compressed by the bulk path) needs its slots zero-filled once before the first append.
 *          Appending one position twice folds that token in twice.
 *   kv_dtype LCS_KV_BF16: win [B, win_ld, c] and kv_out [B, kv_ld, c] bf16 (win_scale, kv_scale
 *          unused); LCS_KV_FP8: the same rows as E4M3FN codes (uint8) with one scale absmax/448 per
 *          row in win_scale [B, win_ld] / kv_scale [B, kv_ld] fp32 (the quantiser of kv_quantize_fp8
 *          applied to the fp32 row).  win_ld >= ring_cap >= 1;
 *   ik_out [B, ik_ld, dI], ik_scale [B, ik_ld] fp32 (fp8).  Rows past kv_ld / ik_ld are not written.
 *   Requirements: c = 512, m >= 1, 0 <= overlap <= m, dI in {64, 128}.
 *   Calls for the same state must be ordered (one stream); concurrent calls on one state race.
 */
size_t kv_decode_state_bytes(int B);
int kv_decode_append(const uint16_t* kv_tok, const float* kv_score,
                     const uint16_t* ik_tok, const float* ik_score,
                     const int64_t* pos, int B, int m, int overlap, int c, int dI,
                     const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset,
                     float* state, size_t state_bytes, int kv_dtype,
                     void* win, float* win_scale, int64_t win_ld, int64_t ring_cap,
                     void* kv_out, float* kv_scale, int64_t kv_ld, int64_t kv_ring,
                     void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype,
                     void* stream);

/*
 * kv_quantize_fp8 -- fp8 storage of K=V rows (page 2, on HCA's mixed FP4 + FP8 precision: the KV
 * cache in FP8 halves its memory): each of `rows` 512-dim bf16 rows becomes E4M3FN codes with one
 * scale absmax/448 (1 for an all-zero row), code = RNE(v / scale) saturating at +-448, with the
 * scale and the division in fp32 (the indexer keys' quantiser).
 *   kv [rows, 512] bf16 (16-byte aligned), codes [rows, 512] uint8 (16-byte aligned), scales [rows].
 */
int kv_quantize_fp8(const uint16_t* kv, int64_t rows, uint8_t* codes, float* scales, void* stream);

/*
 * csa_attend_kv8 / hca_attend_kv8 -- csa_attend / hca_attend on fp8 K=V storage: the cache and the
 * window ring hold E4M3FN codes with one fp32 scale per row (kv_quantize_fp8, or kv_decode_append
 * with LCS_KV_FP8).  Key j is s_j * code_j: its logit is s_j (qhat . code_j) * scale, and
 * o = sum_j p_j s_j code_j / (e^{z} + sum_j p_j); the codes are converted exactly to bf16 for the
 * same MFMA path, so only the storage is fp8.  Arguments as csa_attend / hca_attend with
 *   kv_codes [B, kv_ld, 512] uint8 + kv_scale [B, kv_ld] fp32,
 *   win_codes [B, win_ld, 512] uint8 + win_scale [B, win_ld] fp32 (16-byte aligned codes).
 */
int csa_attend_kv8(const uint16_t* q, const uint16_t* gamma_q, const uint8_t* kv_codes, const float* kv_scale,
                   int64_t kv_ld, const int32_t* topk_idx, int k, const uint8_t* win_codes, const float* win_scale,
                   int64_t win_ld, int64_t ring_cap, int window, const float* sink, const int64_t* q_pos,
                   int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
                   uint16_t* out, void* ws, size_t ws_bytes, void* stream);
int hca_attend_kv8(const uint16_t* q, const uint16_t* gamma_q, const uint8_t* kv_codes, const float* kv_scale,
                   int64_t kv_ld, int64_t n_cap, int m, const uint8_t* win_codes, const float* win_scale,
                   int64_t win_ld, int64_t ring_cap, int window, const float* sink, const int64_t* q_pos,
                   int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
                   uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * hca_attend_append -- an HCA decode step's append and attention in one call (page 1, HCA paragraph:
 * the token is pooled into the compressed state and attends over every visible entry and its window):
 * kv_decode_append with the 29 arguments after ws_bytes (m and overlap: the HCA block size and 0;
 * ik_tok may be NULL), and hca_attend (bf16) or hca_attend_kv8 (kv_dtype = LCS_KV_FP8) over the
 * stores that append writes: cache kv_out / kv_scale with kv_ld, ring win / win_scale with win_ld and
 * ring_cap, block size m.  The result is bit for bit that of kv_decode_append followed by the
 * attention.  The append's workgroups run in the attention's launch; the split holding a query's own
 * token (the window's last key) forms that row as the append does, instead of reading the ring row
 * the append is writing.  Requirements: Tq = 1, B_app = B, kv_ring = 0, and pos[b] equal to
 * q_pos[b, 0] or negative (inactive: the query then reads its window from the ring as stored);
 * otherwise as the two entry points.  Every argument is checked before anything is enqueued.
 */
int hca_attend_append(const uint16_t* q, const uint16_t* gamma_q, int64_t n_cap, int window, const float* sink,
                      const int64_t* q_pos, int64_t rope_offset, int B, int Tq, int H, int c, float scale, float eps,
                      float rope_theta, uint16_t* out, void* ws, size_t ws_bytes,
                      const uint16_t* kv_tok, const float* kv_score, const uint16_t* ik_tok, const float* ik_score,
                      const int64_t* pos, int B_app, int m, int overlap, int c_app, int dI,
                      const uint16_t* gamma_kv, float eps_kv, float rope_theta_kv, int64_t rope_offset_kv,
                      float* state, size_t state_bytes, int kv_dtype,
                      void* win, float* win_scale, int64_t win_ld, int64_t ring_cap,
                      void* kv_out, float* kv_scale, int64_t kv_ld, int64_t kv_ring,
                      void* ik_out, float* ik_scale, int64_t ik_ld, int ik_dtype, void* stream);

/*
 * mhc_sinkhorn -- the doubly stochastic projection of mHC (page 1, section on mHC: the mixing
 * matrix of the residual streams is held on the doubly stochastic matrices by Sinkhorn-Knopp,
 * alternating row and column normalisation, 20 rounds per layer; page 4 section 3.2).  For each of
 * T matrices: M = exp(logits), then `iters` rounds of (every row / its sum, every column / its
 * sum).  fp32 throughout.
 *   logits [T, n, n] fp32 (row-major), b_out [T, n, n] fp32.  1 <= n <= 8, 1 <= iters <= 10000.
 */
int mhc_sinkhorn(const float* logits, int T, int n, int iters, float* b_out, void* stream);

/*
 * mhc_mix -- one mHC residual update of the n streams and the next layer's input, per token
 * (page 1, section on mHC: streams mixed by B, the layer output spread by the output map C and the
 * layer input taken by the input map A, both through a sigmoid).  For token t:
 *   B = mhc_sinkhorn(logits[t, 0 : n*n]),  C = sigmoid(logits[t, n*n : n*n+n]),
 *   A = sigmoid(logits[t, n*n+n : n*n+2n])  (the next layer's input map),
 *   x_out[t, i] = sum_j B_ij x[t, j] + C_i y[t]   (bf16, rounded to nearest even),
 *   h_out[t]    = sum_i A_i x_out[t, i]            (from x_out before its rounding; h_out NULL: skipped).
 *   x, x_out [T, n, d] bf16 (x_out may be x: in place), y, h_out [T, d] bf16,
 *   logits [T, n*n + 2n] fp32.  1 <= n <= 8, d % 8 == 0, 1 <= iters <= 10000; 16-byte aligned.
 */
int mhc_mix(const uint16_t* x, const uint16_t* y, const float* logits, int T, int n, int d, int iters,
            uint16_t* x_out, uint16_t* h_out, void* stream);

/*
 * csa_index_topk -- CSA step 2 (page 1, CSA step 2: lightning indexer + top-k; page 4 section 3.1:
 * 64 indexer heads of dim 128, top-k 512): for each query at token t = q_pos[b, tq] the score of
 * every visible entry s < n_vis = min(t / m, n_cap) is I_s = sum_h w_h * max(0, q_h . k_s); the
 * min(k, n_vis) largest (ties to the lower index) are written ascending, padded with -1.
 * fp8 mode quantises each query head row to E4M3FN (scale absmax/448, round to nearest even,
 * computed in fp32) and multiplies codes on the fp8 matrix cores; accumulation is fp32.
 *
 *   q_idx  [B, Tq, H_I, dI] bf16;  w_idx [B, Tq, H_I] bf16
 *   ik_cache [B, ik_ld, dI] (codes or bf16), ik_scale [B, ik_ld] fp32 (fp8), n_cap <= ik_ld
 *   q_pos  [B, Tq] int64 (device)
 *   topk_idx [B, Tq, k] int32; topk_score [B, Tq, k] fp32 (may be NULL; -inf where padded)
 *   ws     device workspace of at least csa_index_topk_workspace(B, Tq, n_cap, k) bytes, zero-filled
 *          before the first call that uses it.  Every call that returns LCS_OK leaves the workspace's
 *          leading csa_index_topk_state_bytes() bytes zero-filled again (the decode selection's
 *          histograms are cleared by the call's last kernel), so one workspace serves any sequence of
 *          calls, of any shapes, without further clearing; calls that share a workspace must be
 *          ordered (one stream).
 *   Many-row calls (prefill) whose score and candidate rows would exceed 64 MiB for all queries
 *   (B * Tq * n_cap' * 12 bytes, n_cap' = n_cap rounded up to a multiple of 64) score and select
 *   batches of query positions, tb = min(Tq, max(16, 768 / B rounded down to a multiple of 16)) of
 *   every batch row at a time, so the workspace holds B * tb score and candidate rows, not B * Tq.
 *   Requirements: H_I <= 64, dI in {64, 128} (fp8: 128), 1 <= k <= 2048, m >= 1, B * Tq <= 65535 * 16,
 *   and launch grids within the device limits (many-row calls: B * ceil(tb / 16) <= 65535 with bf16
 *   keys, about B <= 65000 with fp8 keys); otherwise LCS_ERR_UNSUPPORTED before anything runs.
 */
size_t csa_index_topk_workspace(int B, int Tq, int64_t n_cap, int k);
size_t csa_index_topk_state_bytes(void);
int csa_index_topk(const uint16_t* q_idx, const uint16_t* w_idx,
                   const void* ik_cache, const float* ik_scale, int64_t ik_ld, int ik_dtype,
                   const int64_t* q_pos, int64_t n_cap,
                   int B, int Tq, int H_I, int dI, int m, int k,
                   int32_t* topk_idx, float* topk_score,
                   void* ws, size_t ws_bytes, void* stream);

/*
 * csa_index_topk_append -- csa_index_topk and kv_decode_append in one call, for a CSA decode step
 * (page 1, CSA steps 1 and 2: the step's new token is pooled into the compressed state while the
 * query selects among the entries visible to it).  The first 18 arguments are csa_index_topk's, the
 * next 29 kv_decode_append's (B_app, m_app, dI_app: its B, m, dI; ik_out, ik_out_scale, ik_out_ld,
 * ik_out_dtype: its ik_out, ik_scale, ik_ld, ik_dtype), then the stream.  Every argument is checked as
 * the two entry points check it, all before anything is enqueued.  The result is that of
 * csa_index_topk followed by kv_decode_append: the append runs beside the selection's last kernel
 * (decode: B * Tq < 64 rows; one launch fewer) or after it (otherwise), once the indexer keys have
 * been scored.  When each sequence's appended token is its query token (pos[b] = q_pos[b, Tq - 1]),
 * the entry a token finishes lies past the entries visible to that query, so the result is also that
 * of the two calls in the other order (the usual decode step: append, then select).  The append's
 * buffers must not overlap the selection's workspace or outputs; ik_out may be ik_cache and pos may
 * be q_pos.
 */
int csa_index_topk_append(const uint16_t* q_idx, const uint16_t* w_idx,
                          const void* ik_cache, const float* ik_scale, int64_t ik_ld, int ik_dtype,
                          const int64_t* q_pos, int64_t n_cap,
                          int B, int Tq, int H_I, int dI, int m, int k,
                          int32_t* topk_idx, float* topk_score,
                          void* ws, size_t ws_bytes,
                          const uint16_t* kv_tok, const float* kv_score,
                          const uint16_t* ik_tok, const float* ik_score,
                          const int64_t* pos, int B_app, int m_app, int overlap, int c, int dI_app,
                          const uint16_t* gamma_kv, float eps, float rope_theta, int64_t rope_offset,
                          float* state, size_t state_bytes, int kv_dtype,
                          void* win, float* win_scale, int64_t win_ld, int64_t ring_cap,
                          void* kv_out, float* kv_scale, int64_t kv_ld, int64_t kv_ring,
                          void* ik_out, float* ik_out_scale, int64_t ik_out_ld, int ik_out_dtype,
                          void* stream);

/*
 * csa_attend -- CSA step 3 (page 1, CSA step 3: multi-query attention over the selected entries;
 * Q/KV normalization; partial RoPE with the -i output rotation; sliding window; sink):
 * per query, qhat_h = RoPE_t(RMSNorm_gamma_q(q_h)); keys = the selected entries of kv_cache
 * (topk_idx >= 0) plus window tokens [t-window+1, t] read from win_ring; K = V.
 *
 *   q [B, Tq, H, c] bf16 raw;  gamma_q [c] bf16
 *   kv_cache [B, kv_ld, c] bf16 (normed + rotated entries); topk_idx [B, Tq, k] int32
 *   win_ring [B, win_ld, c] bf16 (normed + rotated tokens): token j at row j (ring_cap = 0) or
 *            j % ring_cap; the caller keeps every window token of every query present.
 *   sink [H] fp32;  q_pos [B, Tq] int64 (device)
 *   out [B, Tq, H, c] bf16
 *   ws     device workspace of at least lcs_attend_workspace(B, Tq, H, k + window) bytes
 *   Requirements: c = 512, 1 <= H <= 64, window >= 0, k <= 2048.
 */
size_t lcs_attend_workspace(int B, int Tq, int H, int64_t max_keys);
int csa_attend(const uint16_t* q, const uint16_t* gamma_q,
               const uint16_t* kv_cache, int64_t kv_ld, const int32_t* topk_idx, int k,
               const uint16_t* win_ring, int64_t win_ld, int64_t ring_cap, int window,
               const float* sink, const int64_t* q_pos, int64_t rope_offset,
               int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
               uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * hca_attend -- HCA core attention (page 1, HCA paragraph: dense attention over every compressed
 * entry): as csa_attend, but the compressed keys are all visible entries 0 .. n_vis-1 with
 * n_vis = min(t / m, n_cap).  With m = 4 on a CSA cache this is CSA with top-k >= n_vis.
 * Workspace: lcs_attend_workspace(B, Tq, H, n_cap + window).
 */
int hca_attend(const uint16_t* q, const uint16_t* gamma_q,
               const uint16_t* kv_cache, int64_t kv_ld, int64_t n_cap, int m,
               const uint16_t* win_ring, int64_t win_ld, int64_t ring_cap, int window,
               const float* sink, const int64_t* q_pos, int64_t rope_offset,
               int B, int Tq, int H, int c, float scale, float eps, float rope_theta,
               uint16_t* out, void* ws, size_t ws_bytes, void* stream);

/*
 * grouped_out_proj -- CSA step 4 (page 1, CSA step 4: the n_h heads are split into g groups, each
 * group projected to d_g, and the concatenation projected to d):
 *   z[:, j*d_g:(j+1)*d_g] = o[:, heads of group j] . W_g[j]^T   (rounded to bf16)
 *   y = z . W_o^T
 *   o [M, H*c] bf16;  w_g [g, d_g, (H/g)*c] bf16;  w_o [d, g*d_g] bf16;  y [M, d] bf16
 *   ws: grouped_out_proj_workspace(M, g, d_g) bytes (holds z).
 *   Requirements: H % g == 0, d_g % 16 == 0, d % 16 == 0, (H/g)*c % 32 == 0.
 */
size_t grouped_out_proj_workspace(int M, int g, int d_g);
int grouped_out_proj(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o,
                     int M, int H, int c, int g, int d_g, int d, uint16_t* y,
                     void* ws, size_t ws_bytes, void* stream);

/*
 * grouped_out_proj_residual -- grouped_out_proj with the residual stream added: y = z . W_o^T + resid
 * (summed in fp32, rounded once), so consecutive layers chain as h_{l+1} = h_l + layer_l(h_l).
 *   resid [M, d] bf16 (16-byte aligned); resid may be y (in place).  Other arguments as above.
 */
int grouped_out_proj_residual(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o, const uint16_t* resid,
                              int M, int H, int c, int g, int d_g, int d, uint16_t* y, void* ws, size_t ws_bytes,
                              void* stream);

/*
 * grouped_out_proj_noalloc -- grouped_out_proj for callers that cannot allocate device memory
 * (code under HIP graph capture, tight serving loops, harnesses that forbid hipMalloc): the same
 * kernels and the same result, bit for bit, but z lives in a static device array of the library
 * (grouped_out_proj_noalloc_max_bytes() bytes, 4 MiB, held on each GPU the library runs on until the
 * process ends) instead of a caller workspace.  The call allocates and frees nothing; on its first
 * call on a device it looks up that array's device address (the device must be current).
 *   Arguments and requirements as grouped_out_proj (no workspace).  M * g * d_g * 2 bytes, rounded
 *   up to 256, must fit the array, else LCS_ERR_SCRATCH (e.g. M <= 256 at g * d_g = 8192).
 *   Every call on one GPU uses the same array: calls that may overlap on one GPU (other streams,
 *   other threads) race and must be ordered by the caller.
 */
size_t grouped_out_proj_noalloc_max_bytes(void);
int grouped_out_proj_noalloc(const uint16_t* o, const uint16_t* w_g, const uint16_t* w_o,
                             int M, int H, int c, int g, int d_g, int d, uint16_t* y, void* stream);

/*
 * input_proj -- the layer's input projections from the hidden state in one pass over their
 * concatenated weights (upstream of page 1's CSA steps: the query heads, the per-token K=V vector and
 * pooling logit, the indexer's query heads, head weights, key and key logit are all linear maps of
 * the token's hidden state h): out = h . W_in^T, with the output columns split into segments.
 *   h [M, d] bf16 (M <= 8 rows: decode; d = 4096 or 8192), w_in [n_rows, d] bf16 output-major,
 *   n_rows % 16 == 0 (pad with rows whose outputs fall past the last segment).
 *   Segment s (n_seg <= 8) takes the next seg_width[s] columns and writes them to seg_dst[s] as
 *   row-major [M, seg_ld[s]] (seg_ld[s] >= seg_width[s]), fp32 if seg_fp32[s] else bf16 (RNE).
 *   seg_* are host arrays; seg_dst[s] are device pointers.
 */
int input_proj(const uint16_t* h, int M, int d, const uint16_t* w_in, int n_rows, int n_seg, const int* seg_width,
               void* const* seg_dst, const int64_t* seg_ld, const int* seg_fp32, void* stream);

/*
 * Kernel timing (measurement facility, off by default).  While enabled, every kernel launch made
 * by the library is bracketed by two hipEvents recorded on the launch stream; lcs_timing_read
 * synchronises those events and returns the summed duration and launch count of the kernels whose
 * name contains `name`.  Not for use under stream capture.  lcs_timing_enable(0) drops the events.
 * This is the part of the ABI that keeps process-wide state (the recorded events, under a mutex)
 * and synchronises with the device (lcs_timing_read waits for the events it reads); it exists so a
 * benchmark can time each kernel on the stream it was launched on.  The events are created with
 * hipEventDisableSystemFence, so recording one adds no cache write-back or invalidation between
 * the launches it brackets.  While disabled, a launch pays one relaxed atomic load.
 */
int lcs_timing_enable(int on);
int lcs_timing_read(const char* name, double* total_ms, int64_t* launches);

#ifdef __cplusplus
}
#endif
#endif /* LCS_H_ */
