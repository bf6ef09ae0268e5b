"""Plain, slow fp64 CPU oracle of the DeepSeek-V4 hybrid compressed attention forward.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path imports this module;
only the tests, the smoke check and the benchmark's CPU-baseline leg do.  It
shares no code with the HIP library.

Sources (cited by page and section; the pages are web articles on the V4 release):
  [P1 hybrid]  page 1, "DeepSeek V4 ..." walk-through (gxgjx.lffhtl.com/lxrt/355279.html),
               section 混合注意力机制 ("hybrid attention"): the four CSA steps, HCA, Q/KV RMSNorm,
               partial RoPE with the output rotation by -i, the sliding-window branch, the sink.
  [P4 3.1]     page 4, "DeepSeek-V4开源解读" (zhinnengdao.top), section 3.1 "Hybrid Attention:
               CSA + HCA": Flash constants m = 4, indexer 64 heads x 128, top-k 512, m' = 128,
               RoPE on the last 64 dims, one sink logit per head, a window branch per layer type.
  [OFP8]       the OCP 8-bit floating point specification (E4M3FN), for the fp8 code table.
  [P1 mHC]     page 1, section on mHC (给残差集结加层连续, "a constraint on the residual connection"):
               n_hc parallel residual streams mixed by a matrix B constrained to the doubly
               stochastic matrices (rows and columns sum to 1) by Sinkhorn-Knopp, alternating row and
               column normalisation for 20 iterations per layer; input map A and output map C passed
               through a sigmoid.
  [P4 3.2]     page 4, section 3.2 "mHC": the residual mapping constrained to the doubly stochastic
               manifold; parameters generated dynamically (input-dependent and input-independent parts).

Readings where the pages are silent (each is listed in the design doc):
  R1  pooling logits are one scalar per token, given as input; softmax over the block window.
  R2  CSA overlap ov = m: block i pools tokens [i*m - ov, (i+1)*m), tokens < 0 dropped.
  R3  RMSNorm after pooling (and on each window token, and per query head), eps 1e-6, then RoPE.
  R4  RoPE on dims 448..511 as adjacent pairs, angle p * theta^(-j/32), theta = 10000; entry i is
      placed at position (i+1)*m - 1, window token j at j, query t at t; output rotated by -t.
  R5  logits scaled by 1/sqrt(512); the sink z_h adds exp(z_h) to the denominator only.
  R6  entry i is visible to query t iff (i+1)*m <= t  (n_vis = t // m).
  R7  window = tokens [max(0, t-W+1), t], self included; one joint softmax with the compressed keys.
  R8  indexer score I_s = sum_h w_h * relu(q_h . k_s); fp8 mode quantises q rows and k entries to
      E4M3FN with a per-row absmax/448 scale; top-k ties go to the lower index; ascending, -1 padded.
  R9  grouped projection: group j = heads [j*H/g, (j+1)*H/g); z_j = o_group . W_g[j]^T; y = z . W_o^T
      (weights stored output-major, [out, in]).
  R11 input projections (upstream of [P1 hybrid] CSA steps 1-3: the query heads, the per-token K=V
      vector and pooling logit, the indexer's query heads, head weights, key and key logit are linear
      maps of the token's hidden state h): one output-major matrix per output, concatenated; the
      layers of a stack chain through the residual h_{l+1} = h_l + y_l.
  R10 mHC: per token the mixing logits are given (their generation from the streams is a projection
      upstream of the kernel); B = Sinkhorn-Knopp of exp(logits), each round dividing every row by
      its sum and then every column by its sum; A = sigmoid, C = sigmoid; the streams update as
      X'_i = sum_j B_ij X_j + C_i y and the next layer's input is h = sum_i A_i X'_i.

All arithmetic is float64 unless a function says it follows the kernel's precision to take the
same integer decision (fp8 codes of the query rows).
"""
from __future__ import annotations

import math

import numpy as np

C_HEAD = 512          # head dim c  [P1 hybrid] (V4 sets c = 512)
ROPE_DIMS = 64        # RoPE on the last 64 dims [P1 hybrid], [P4 3.1]
ROPE_START = C_HEAD - ROPE_DIMS
E4M3_MAX = 448.0      # [OFP8] largest finite E4M3FN magnitude


# ---------------------------------------------------------------------------------------------
# Normalisation and rotary position encoding
# ---------------------------------------------------------------------------------------------
def rmsnorm(x, gamma, eps):
    """RMSNorm over the last axis [P1 hybrid, "Q/KV normalization"]: gamma * x / sqrt(mean(x^2)+eps)."""
    x = np.asarray(x, dtype=np.float64)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return np.asarray(gamma, dtype=np.float64) * x / np.sqrt(ms + eps)


def rope_angles(pos, theta=10000.0):
    """Angles p * theta^(-j/32) for the 32 rotated pairs (reading R4), in float64."""
    j = np.arange(ROPE_DIMS // 2, dtype=np.float64)
    inv = np.power(float(theta), -j / (ROPE_DIMS // 2))
    return float(pos) * inv


def rope(x, pos, theta=10000.0):
    """Rotate the last 64 dims of a c=512 vector by position ``pos`` [P1 hybrid, "Partial RoPE"].

    Pairs are (448+2j, 449+2j): (a, b) -> (a cos f - b sin f, a sin f + b cos f).
    Dims 0..447 pass through unchanged.
    """
    y = np.array(x, dtype=np.float64, copy=True)
    phi = rope_angles(pos, theta)
    cs, sn = np.cos(phi), np.sin(phi)
    a = y[..., ROPE_START::2].copy()
    b = y[..., ROPE_START + 1::2].copy()
    y[..., ROPE_START::2] = a * cs - b * sn
    y[..., ROPE_START + 1::2] = a * sn + b * cs
    return y


# ---------------------------------------------------------------------------------------------
# Step 1: learned softmax-pooling KV compression  [P1 hybrid, CSA step 1; HCA paragraph]
# ---------------------------------------------------------------------------------------------
def block_span(i, m, ov):
    """Token range [lo, hi) pooled into entry i (readings R2/R3)."""
    return max(0, i * m - ov), (i + 1) * m


def pool(x_tok, s_tok, m, ov, n_blk=None):
    """Entry i = sum_j softmax(s[S_i])_j x_j over S_i = [i*m-ov, (i+1)*m) (reading R1).

    x_tok [T, D], s_tok [T]; returns [n_blk, D] with n_blk = T // m by default.
    """
    x = np.asarray(x_tok, dtype=np.float64)
    s = np.asarray(s_tok, dtype=np.float64)
    T = x.shape[0]
    if n_blk is None:
        n_blk = T // m
    out = np.zeros((n_blk, x.shape[1]), dtype=np.float64)
    for i in range(n_blk):
        lo, hi = block_span(i, m, ov)
        logits = s[lo:hi]
        a = np.exp(logits - logits.max())
        a = a / a.sum()
        out[i] = a @ x[lo:hi]
    return out


def entry_position(i, m):
    """Position an entry is rotated to: the last token of its block (reading R4)."""
    return (i + 1) * m - 1


def compress_kv(x_tok, s_tok, m, ov, gamma, eps=1e-6, theta=10000.0, rope_offset=0):
    """Compressed K=V entries: pool, RMSNorm, then RoPE at (i+1)*m-1+offset (readings R2-R4)."""
    e = pool(x_tok, s_tok, m, ov)
    out = np.empty_like(e)
    for i in range(e.shape[0]):
        out[i] = rope(rmsnorm(e[i], gamma, eps), entry_position(i, m) + rope_offset, theta)
    return out


def window_entries(x_tok, gamma, eps=1e-6, theta=10000.0, rope_offset=0):
    """Uncompressed window keys: each token RMSNorm'd and rotated to its own position (m = 1)."""
    x = np.asarray(x_tok, dtype=np.float64)
    return np.stack([rope(rmsnorm(x[j], gamma, eps), j + rope_offset, theta) for j in range(x.shape[0])]) \
        if x.shape[0] else np.zeros((0, x.shape[1]))


# ---------------------------------------------------------------------------------------------
# fp8 E4M3FN  [OFP8]; used for the indexer keys and queries (reading R8)
# ---------------------------------------------------------------------------------------------
def e4m3_value(code):
    """Value of one E4M3FN byte: s eeee mmm, bias 7; e=0 subnormal m*2^-9; 0x7F/0xFF NaN."""
    code = int(code) & 0xFF
    sign = -1.0 if code & 0x80 else 1.0
    e = (code >> 3) & 0xF
    mm = code & 0x7
    if e == 15 and mm == 7:
        return float("nan")
    if e == 0:
        return sign * mm * 2.0 ** -9
    return sign * (1.0 + mm / 8.0) * 2.0 ** (e - 7)


_E4M3_POS = np.array([e4m3_value(c) for c in range(127)], dtype=np.float64)   # codes 0..126


def e4m3_table():
    """The 127 finite non-negative E4M3FN values, indexed by code (increasing in the code)."""
    return _E4M3_POS.copy()


def e4m3_encode(v):
    """Nearest E4M3FN code of each value; ties to the even code; saturates at +-448.

    Works on the exact (float64) value of the input, so float32 inputs round once.
    """
    v = np.asarray(v, dtype=np.float64)
    a = np.minimum(np.abs(v), E4M3_MAX)
    hi = np.searchsorted(_E4M3_POS, a, side="left")          # first table value >= a
    hi = np.clip(hi, 0, 126)
    lo = np.clip(hi - 1, 0, 126)
    d_hi = _E4M3_POS[hi] - a
    d_lo = a - _E4M3_POS[lo]
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.int64)
    code = np.where(a == _E4M3_POS[hi], hi, code)
    neg = (v < 0) & (code != 0)
    return (code | (neg.astype(np.int64) << 7)).astype(np.uint8)


def e4m3_decode(codes):
    c = np.asarray(codes, dtype=np.int64)
    mag = _E4M3_POS[np.minimum(c & 0x7F, 126)]
    return np.where(c & 0x80, -mag, mag)


def fp8_quantize_rows(v, kernel_fp32=False):
    """Per-row absmax scaling to 448 and E4M3FN rounding (reading R8).

    Returns (codes [.., D] uint8, scale [..] float, dequantised float64).
    scale = absmax/448 (1 where absmax = 0).  With ``kernel_fp32`` the scale and v/scale are
    formed in float32 (IEEE division), so the code decision is taken in the GPU kernel's precision.
    """
    v = np.asarray(v, dtype=np.float64)
    amax = np.max(np.abs(v), axis=-1)
    if kernel_fp32:
        a32 = amax.astype(np.float32)
        s = np.where(a32 > 0, a32 / np.float32(E4M3_MAX), np.float32(1.0)).astype(np.float32)
        q = (v.astype(np.float32) / s[..., None]).astype(np.float32)
        codes = e4m3_encode(q.astype(np.float64))
        s64 = s.astype(np.float64)
    else:
        s64 = np.where(amax > 0, amax / E4M3_MAX, 1.0)
        codes = e4m3_encode(v / s64[..., None])
    return codes, s64, e4m3_decode(codes) * s64[..., None]


def compress_ik(ik_tok, ik_score, m, ov, fp8=True):
    """Indexer keys: pooled like the KV entries with their own logits; no norm, no RoPE (reading R8).

    fp8: returns (codes, scales, dequantised); bf16 mode returns the pooled float64 keys.
    """
    e = pool(ik_tok, ik_score, m, ov)
    if fp8:
        return fp8_quantize_rows(e)
    return e


# ---------------------------------------------------------------------------------------------
# Steps 2: lightning indexer + top-k  [P1 hybrid, CSA step 2], [P4 3.1]
# ---------------------------------------------------------------------------------------------
def n_visible(t, m):
    """Entries a query at token t may see: i with (i+1)*m <= t (reading R6)."""
    return t // m


def index_scores(q_idx, w_idx, k_idx):
    """I_s = sum_h w_h * max(0, q_h . k_s) for every entry s given (reading R8).

    q_idx [H_I, d_I], w_idx [H_I], k_idx [n, d_I] -> [n]
    """
    q = np.asarray(q_idx, dtype=np.float64)
    w = np.asarray(w_idx, dtype=np.float64)
    k = np.asarray(k_idx, dtype=np.float64)
    dots = k @ q.T                                 # [n, H_I]
    return np.maximum(dots, 0.0) @ w


def topk_select(scores, k):
    """First min(k, n) of a stable sort by (-score, index); returned ascending, padded with -1."""
    s = np.asarray(scores, dtype=np.float64)
    n = s.shape[0]
    order = np.lexsort((np.arange(n), -s))          # primary -score, secondary index
    sel = np.sort(order[: min(k, n)])
    out = -np.ones(k, dtype=np.int64)
    out[: sel.shape[0]] = sel
    return out


# ---------------------------------------------------------------------------------------------
# Step 3: core MQA over the selected entries plus the window, with the sink [P1 hybrid]
# ---------------------------------------------------------------------------------------------
def attend_one(q_heads, gamma_q, keys, sink, t, scale, eps=1e-6, theta=10000.0, rope_offset=0):
    """Output of every head for one query at token t over the key set ``keys`` (K = V).

    q_heads [H, 512] raw; keys [n, 512] already normalised and rotated; sink [H].
    q_h <- rope(rmsnorm(q_h), t); l = scale * K q_h; p = e^l / (e^z + sum e^l); o = p K;
    then the last 64 dims of o are rotated by -(t) (readings R3-R5, R7).
    """
    q = np.asarray(q_heads, dtype=np.float64)
    K = np.asarray(keys, dtype=np.float64)
    H = q.shape[0]
    out = np.zeros((H, q.shape[1]), dtype=np.float64)
    for h in range(H):
        qh = rope(rmsnorm(q[h], gamma_q, eps), t + rope_offset, theta)
        z = float(sink[h])
        if K.shape[0] == 0:
            continue
        logit = scale * (K @ qh)
        M = max(float(logit.max()), z)
        e = np.exp(logit - M)
        den = e.sum() + (math.exp(z - M) if z != -math.inf else 0.0)
        o = (e / den) @ K
        out[h] = rope(o, -(t + rope_offset), theta)
    return out


def window_range(t, W):
    return max(0, t - W + 1), t + 1


def csa_attend_one(q_heads, gamma_q, kv_entries, sel, win_keys_all, sink, t, W, scale,
                   eps=1e-6, theta=10000.0, rope_offset=0):
    """CSA: keys = selected compressed entries (indices >= 0 of ``sel``) ++ window tokens."""
    sel = [int(s) for s in sel if s >= 0]
    lo, hi = window_range(t, W)
    ent = np.asarray(kv_entries, dtype=np.float64)
    chosen = ent[sel] if sel else np.zeros((0, ent.shape[1]))
    keys = np.concatenate([chosen, np.asarray(win_keys_all, dtype=np.float64)[lo:hi]], axis=0)
    return attend_one(q_heads, gamma_q, keys, sink, t, scale, eps, theta, rope_offset)


def hca_attend_one(q_heads, gamma_q, kv_entries, m, win_keys_all, sink, t, W, scale,
                   eps=1e-6, theta=10000.0, rope_offset=0):
    """HCA: keys = every visible compressed entry (n_vis = t // m) ++ window tokens."""
    n = min(n_visible(t, m), np.asarray(kv_entries).shape[0])
    lo, hi = window_range(t, W)
    keys = np.concatenate([np.asarray(kv_entries, dtype=np.float64)[:n],
                           np.asarray(win_keys_all, dtype=np.float64)[lo:hi]], axis=0)
    return attend_one(q_heads, gamma_q, keys, sink, t, scale, eps, theta, rope_offset)


# ---------------------------------------------------------------------------------------------
# Step 4: grouped output projection [P1 hybrid, CSA step 4] (reading R9)
# ---------------------------------------------------------------------------------------------
def grouped_out_proj(o, w_g, w_o):
    """o [M, H*c]; w_g [g, d_g, (H/g)*c]; w_o [d, g*d_g]  ->  (z [M, g*d_g], y [M, d])."""
    o = np.asarray(o, dtype=np.float64)
    w_g = np.asarray(w_g, dtype=np.float64)
    w_o = np.asarray(w_o, dtype=np.float64)
    g, d_g, kg = w_g.shape
    z = np.concatenate([o[:, j * kg:(j + 1) * kg] @ w_g[j].T for j in range(g)], axis=1)
    return z, z @ w_o.T


# ---------------------------------------------------------------------------------------------
# Textbook causal multi-query attention (for the reduction invariants)
# ---------------------------------------------------------------------------------------------
def causal_mqa(q_tok, gamma_q, kv_tok, gamma_kv, scale, eps=1e-6, theta=10000.0, rope_offset=0):
    """softmax(Qhat Khat^T * scale + causal mask) Khat with the same norm/RoPE and -t output rotation.

    q_tok [T, H, 512], kv_tok [T, 512] raw per-token vectors; no sink.
    """
    q = np.asarray(q_tok, dtype=np.float64)
    T, H, D = q.shape
    K = np.stack([rope(rmsnorm(kv_tok[j], gamma_kv, eps), j + rope_offset, theta) for j in range(T)])
    out = np.zeros_like(q)
    mask = np.triu(np.full((T, T), -np.inf), k=1)
    for h in range(H):
        Q = np.stack([rope(rmsnorm(q[t, h], gamma_q, eps), t + rope_offset, theta) for t in range(T)])
        L = scale * (Q @ K.T) + mask
        L = L - L.max(axis=1, keepdims=True)
        P = np.exp(L)
        P = P / P.sum(axis=1, keepdims=True)
        O = P @ K
        out[:, h] = np.stack([rope(O[t], -(t + rope_offset), theta) for t in range(T)])
    return out


# ---------------------------------------------------------------------------------------------
# Whole layers (one sequence), composed from the steps above in the pages' order
# ---------------------------------------------------------------------------------------------
def csa_layer(kv_tok, kv_score, ik_tok, ik_score, q, q_idx, w_idx, sink, positions, *,
              m=4, ov=4, W=128, k=512, fp8=True, gamma_kv=None, gamma_q=None,
              eps=1e-6, theta=10000.0, rope_offset=0, scale=None):
    """CSA for one sequence: compress -> index -> top-k -> attend at each query position.

    kv_tok [T,512], kv_score [T], ik_tok [T,d_I], ik_score [T]; q [Tq,H,512], q_idx [Tq,H_I,d_I],
    w_idx [Tq,H_I]; positions [Tq] absolute token indices (all < T).
    Returns (o [Tq,H,512], topk [Tq,k], scores list).
    """
    D = np.asarray(kv_tok).shape[1]
    gamma_kv = np.ones(D) if gamma_kv is None else gamma_kv
    gamma_q = np.ones(D) if gamma_q is None else gamma_q
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    entries = compress_kv(kv_tok, kv_score, m, ov, gamma_kv, eps, theta, rope_offset)
    if fp8:
        _, _, kI = compress_ik(ik_tok, ik_score, m, ov, fp8=True)
    else:
        kI = compress_ik(ik_tok, ik_score, m, ov, fp8=False)
    win = window_entries(kv_tok, gamma_kv, eps, theta, rope_offset)
    outs, sels, scs = [], [], []
    for qi, t in enumerate(positions):
        n = n_visible(t, m)
        qI = np.asarray(q_idx[qi], dtype=np.float64)
        if fp8:
            _, _, qI = fp8_quantize_rows(qI)
        sc = index_scores(qI, w_idx[qi], kI[:n])
        sel = topk_select(sc, k)
        outs.append(csa_attend_one(q[qi], gamma_q, entries, sel, win, sink, t, W, scale,
                                   eps, theta, rope_offset))
        sels.append(sel)
        scs.append(sc)
    return np.stack(outs), np.stack(sels), scs


def hca_layer(kv_tok, kv_score, q, sink, positions, *, m=128, W=128, gamma_kv=None, gamma_q=None,
              eps=1e-6, theta=10000.0, rope_offset=0, scale=None):
    """HCA for one sequence: non-overlapping m-token compression then dense attention [P1 hybrid]."""
    D = np.asarray(kv_tok).shape[1]
    gamma_kv = np.ones(D) if gamma_kv is None else gamma_kv
    gamma_q = np.ones(D) if gamma_q is None else gamma_q
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    entries = compress_kv(kv_tok, kv_score, m, 0, gamma_kv, eps, theta, rope_offset)
    win = window_entries(kv_tok, gamma_kv, eps, theta, rope_offset)
    return np.stack([hca_attend_one(q[qi], gamma_q, entries, m, win, sink, t, W, scale,
                                    eps, theta, rope_offset) for qi, t in enumerate(positions)])


# ---------------------------------------------------------------------------------------------
# mHC: mixing of the n_hc residual streams  [P1 mHC], [P4 3.2]
# ---------------------------------------------------------------------------------------------
MHC_ITERS = 20        # Sinkhorn-Knopp rounds per layer [P1 mHC]


def sigmoid(x):
    """The map that keeps A and C non-negative and bounded [P1 mHC]."""
    return 1.0 / (1.0 + np.exp(-np.asarray(x, dtype=np.float64)))


def sinkhorn(logits, iters=MHC_ITERS):
    """Doubly stochastic projection of one n x n matrix of mixing logits [P1 mHC] (R10): start from
    the positive matrix exp(logits); each round divides every row by its sum, then every column by
    its sum (so after any round the columns sum to 1 and the rows approach 1)."""
    M = np.exp(np.asarray(logits, dtype=np.float64))
    for _ in range(iters):
        M = M / M.sum(axis=1, keepdims=True)
        M = M / M.sum(axis=0, keepdims=True)
    return M


def mhc_mix(X, y, logits, iters=MHC_ITERS):
    """One residual update of the n streams and the next layer's input, per token [P1 mHC] (R10).

    X [T, n, d] streams; y [T, d] the layer's output; logits [T, n*n + 2n] per token: the mixing
    logits (row-major), then the output-map logits C~, then the next layer's input-map logits A~.
    Returns (X' [T, n, d] with X'_i = sum_j B_ij X_j + sigmoid(C~_i) y,  h [T, d] = sum_i sigmoid(A~_i) X'_i).
    """
    X = np.asarray(X, dtype=np.float64)
    y = np.asarray(y, dtype=np.float64)
    L = np.asarray(logits, dtype=np.float64)
    T, n, d = X.shape
    Xo = np.empty((T, n, d))
    h = np.empty((T, d))
    for t in range(T):
        B = sinkhorn(L[t, : n * n].reshape(n, n), iters)
        C = sigmoid(L[t, n * n: n * n + n])
        A = sigmoid(L[t, n * n + n: n * n + 2 * n])
        Xo[t] = B @ X[t] + C[:, None] * y[t][None, :]
        h[t] = A @ Xo[t]
    return Xo, h


# ---------------------------------------------------------------------------------------------
# Input projections and the residual chain of a stack of layers (R11)
# ---------------------------------------------------------------------------------------------
def input_projection(h, w_in, widths):
    """Outputs of a layer's input projections (R11): out = h . W_in^T (W_in output-major,
    [sum(widths) + padding, d]), split into consecutive column groups of the given widths."""
    out = np.asarray(h, dtype=np.float64) @ np.asarray(w_in, dtype=np.float64).T
    parts, c = [], 0
    for w in widths:
        parts.append(out[:, c: c + w])
        c += w
    return parts


def residual(h, y):
    """Residual chaining of consecutive layers (R11): h_{l+1} = h_l + y_l."""
    return np.asarray(h, dtype=np.float64) + np.asarray(y, dtype=np.float64)
