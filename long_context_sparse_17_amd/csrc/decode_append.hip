// One decode step of the compressed-KV state for a batch of sequences, each at its own position
// (page 1, "hybrid attention": CSA step 1, the HCA paragraph and the sliding-window branch).
//
// A token t of sequence b is (1) written to the window ring as RoPE_t(RMSNorm(kv)), (2) folded into
// the pooling state of every block that contains it, and (3) when t is the last token of block i,
// block i's entry is finished: pooled vector RMSNorm'd, rotated to t and stored, with the indexer
// key (own logits, no norm, no RoPE) stored as bf16 or E4M3FN codes + scale.  Ring rows and
// entries are stored as bf16, or (kv8) as E4M3FN codes with one scale absmax / 448 per row.  The pooled vector is
// the same softmax-weighted sum the bulk compression forms, accumulated online as tokens arrive:
// a running max M, sum l = sum e^{s_j - M} and weighted sums acc = sum e^{s_j - M} x_j (fp32),
// rescaled when M grows; entry = acc / l.
//
// With overlap ov <= m a token belongs to block i = t / m and, when t >= (i+1)m - ov, to block
// i + 1, so each sequence keeps two state slots (block j uses slot j & 1), tagged with the block
// they hold.  The first token of a block (max(0, jm - ov)) starts its slot and tag; a later token
// whose slot carries another tag belongs to a block whose first token was never appended (a
// sequence resumed mid-stream): that block is left alone and its entry is not written.
//
// One workgroup of 128 threads per sequence; thread x owns K=V dims 4x .. 4x+3 and indexer dim x.
#include "decode_append.h"

namespace lcs {

namespace {

__global__ void __launch_bounds__(dapp::kThreads)
decode_append_kernel(DecodeAppendArgs a, RopeFreq rf) {
  __shared__ float red[2];
  dapp::decode_append_seq(a, rf, blockIdx.x, red);
}

}  // namespace

size_t decode_state_bytes(int B) { return (size_t)B * 2 * kStateFloats * sizeof(float); }

int launch_decode_append(const DecodeAppendArgs& a, hipStream_t stream) {
  LCS_LAUNCH("decode_append_kernel", decode_append_kernel, dim3((unsigned)a.B), dim3(dapp::kThreads), 0, stream, a,
             rope_freq(a.theta));
  return hipGetLastError() == hipSuccess ? 0 : 4;
}

}  // namespace lcs
