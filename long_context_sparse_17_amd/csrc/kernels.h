// Internal launcher interface between the C-ABI layer and the kernels (not exported).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace lcs {

struct CompressArgs {
  const uint16_t* kv_tok; const float* kv_score; const uint16_t* ik_tok; const float* ik_score;
  int B, T; int64_t tok0, blk_begin; int n_blk, m, ov, dI;
  const uint16_t* gamma; float eps, theta; int64_t rope_offset;
  uint16_t* kv_out; int64_t kv_ld, ring_cap;
  void* ik_out; float* ik_scale; int64_t ik_ld; int ik_fp8;
};
int launch_compress(const CompressArgs& a, hipStream_t stream);

// Decode-step append (per-sequence positions, online pooling state).  State per sequence: two slots
// of kStateFloats floats: K=V weighted sums [512], indexer weighted sums [kMaxIdxDim], then
// (M, l) for the K=V, (M, l) for the indexer logits, and the tag (block index + 1, int32 bits; 0 =
// empty) of the block the slot holds; padded to a multiple of 4 floats.
constexpr int kMaxIdxDim = 128;
constexpr int kStateFloats = 512 + kMaxIdxDim + 8;
struct DecodeAppendArgs {
  const uint16_t* kv_tok; const float* kv_score; const uint16_t* ik_tok; const float* ik_score;
  const int64_t* pos; int B, m, ov, dI;
  const uint16_t* gamma; float eps, theta; int64_t rope_offset;
  float* state;
  void* win; int64_t win_ld, ring_cap;
  void* kv_out; int64_t kv_ld, kv_ring;
  int kv8; float* win_scale; float* kv_scale;   // kv8: ring rows and entries as E4M3FN codes + row scales
  void* ik_out; float* ik_scale; int64_t ik_ld; int ik_fp8;
};
size_t decode_state_bytes(int B);
int launch_decode_append(const DecodeAppendArgs& a, hipStream_t stream);

int launch_kv_quantize(const uint16_t* kv, int64_t rows, uint8_t* codes, float* scales, hipStream_t stream);

// mHC stream mixing (x != nullptr) or the Sinkhorn-Knopp projection alone (x == nullptr).
struct MhcArgs {
  const uint16_t* x; const uint16_t* y; const float* logits;
  int T, n, d, iters;
  uint16_t* x_out; uint16_t* h_out; float* b_out;
};
int launch_mhc(const MhcArgs& a, hipStream_t stream);

struct IndexArgs {
  const uint16_t* q_idx; const uint16_t* w_idx;
  const void* ik; const float* ik_scale; int64_t ik_ld; int ik_fp8;
  const int64_t* q_pos; int64_t n_cap;
  int B, Tq, H_I, dI, m, k;
  int32_t* topk_idx; float* topk_score;
  void* ws; size_t ws_bytes;
  const DecodeAppendArgs* append = nullptr;   // also run this token append (decode: beside the final selection)
};
size_t index_topk_workspace(int B, int Tq, int64_t n_cap, int k);
size_t index_topk_state_bytes();   // leading workspace bytes that stay zero between calls
bool index_topk_launchable(int B, int Tq, int64_t n_cap, int ik_fp8);
int launch_index_topk(const IndexArgs& a, hipStream_t stream);

struct AttendArgs {
  const uint16_t* q; const uint16_t* gamma_q;
  const uint16_t* kv; int64_t kv_ld;
  const uint8_t* kv8; const float* kv_scale;     // fp8 K=V (kv8 != nullptr): codes + per-row scales
  const uint8_t* win8; const float* win_scale;   //   for the cache and the window ring
  const int32_t* topk; int k;          // CSA: selected entries (topk != nullptr)
  int64_t n_cap; int m;                // HCA: all visible entries
  const uint16_t* win; int64_t win_ld, ring_cap; int window;
  const float* sink; const int64_t* q_pos; int64_t rope_offset;
  int B, Tq, H; float scale, eps, theta;
  uint16_t* out; void* ws; size_t ws_bytes;
  // dense visible ranges (HCA) with one query per sequence: also run this token append (pos[b] = the
  // query position or negative), its workgroups in the same launch
  const DecodeAppendArgs* append = nullptr;
};
size_t attend_workspace(int B, int Tq, int H, int64_t max_keys);
bool attend_launchable(int B, int Tq, int H, int64_t max_keys, bool list);
int launch_attend(const AttendArgs& a, int64_t max_keys, hipStream_t stream);

struct OutProjArgs {
  const uint16_t* o; const uint16_t* w_g; const uint16_t* w_o;
  int M, H, c, g, d_g, d; uint16_t* y; void* ws; size_t ws_bytes;
  const uint16_t* resid = nullptr;     // y = z . W_o^T + resid  ([M, d] bf16), nullptr: none
};

// Output segments of a concatenated projection: columns [end[s-1], end[s]) go to dst[s] (row
// stride ld[s] elements, fp32 if f32[s] else bf16); columns past end[n-1] are dropped.
constexpr int kMaxProjSegments = 8;
struct ProjSegments {
  int n;
  int end[kMaxProjSegments];
  void* dst[kMaxProjSegments];
  int64_t ld[kMaxProjSegments];
  int f32[kMaxProjSegments];
};
int launch_input_proj(const uint16_t* h, int M, int d, const uint16_t* w, int n_rows, const ProjSegments& seg,
                      hipStream_t stream);
size_t out_proj_workspace(int M, int g, int d_g);
// Allocation-free variant: z in a static device array of kOutProjScratchBytes (per device).
constexpr size_t kOutProjScratchBytes = (size_t)4 << 20;
int out_proj_scratch(void** ptr);
int launch_out_proj(const OutProjArgs& a, hipStream_t stream);

}  // namespace lcs
