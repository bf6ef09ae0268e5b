"""Python binding of liblcs.so, the gfx950 hybrid compressed attention forward (CSA + HCA).

Argument marshalling only: every step runs in the HIP kernels behind the C ABI declared in
include/lcs.h.  Tensors are torch tensors on the GPU (torch supplies device memory and the
stream); shapes are read off the tensors and passed as plain sizes and pointers.  There is no
fallback: if liblcs.so is missing or fails to load, the functions raise.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "liblcs.so")

LCS_OK, LCS_ERR_ARG, LCS_ERR_UNSUPPORTED, LCS_ERR_WORKSPACE, LCS_ERR_HIP, LCS_ERR_SCRATCH = 0, 1, 2, 3, 4, 5
LCS_IK_BF16, LCS_IK_FP8 = 0, 1
LCS_KV_BF16, LCS_KV_FP8 = 0, 1
HEAD_DIM = 512

# exported symbols and their C signatures (see include/lcs.h)
_P, _I, _I64, _F, _SZ = ctypes.c_void_p, ctypes.c_int, ctypes.c_int64, ctypes.c_float, ctypes.c_size_t
SIGNATURES = {
    "lcs_version": (_I, []),
    "lcs_status_string": (ctypes.c_char_p, [_I]),
    "csa_compress_kv": (_I, [_P, _P, _P, _P, _I, _I, _I64, _I64, _I, _I, _I, _I, _I, _P, _F, _F, _I64,
                             _P, _I64, _I64, _P, _P, _I64, _I, _P]),
    "hca_compress_kv": (_I, [_P, _P, _I, _I, _I64, _I64, _I, _I, _I, _P, _F, _F, _I64, _P, _I64, _I64, _P]),
    "kv_decode_state_bytes": (_SZ, [_I]),
    "kv_decode_append": (_I, [_P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _F, _F, _I64, _P, _SZ, _I, _P, _P, _I64,
                              _I64, _P, _P, _I64, _I64, _P, _P, _I64, _I, _P]),
    "kv_quantize_fp8": (_I, [_P, _I64, _P, _P, _P]),
    "csa_attend_kv8": (_I, [_P, _P, _P, _P, _I64, _P, _I, _P, _P, _I64, _I64, _I, _P, _P, _I64, _I, _I, _I, _I, _F,
                            _F, _F, _P, _P, _SZ, _P]),
    "hca_attend_kv8": (_I, [_P, _P, _P, _P, _I64, _I64, _I, _P, _P, _I64, _I64, _I, _P, _P, _I64, _I, _I, _I, _I, _F,
                            _F, _F, _P, _P, _SZ, _P]),
    "mhc_sinkhorn": (_I, [_P, _I, _I, _I, _P, _P]),
    "mhc_mix": (_I, [_P, _P, _P, _I, _I, _I, _I, _P, _P, _P]),
    "csa_index_topk_workspace": (_SZ, [_I, _I, _I64, _I]),
    "csa_index_topk_state_bytes": (_SZ, []),
    "csa_index_topk": (_I, [_P, _P, _P, _P, _I64, _I, _P, _I64, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ, _P]),
    "hca_attend_append": (_I, [_P, _P, _I64, _I, _P, _P, _I64, _I, _I, _I, _I, _F, _F, _F, _P, _P, _SZ,
                               _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _F, _F, _I64, _P, _SZ, _I, _P, _P,
                               _I64, _I64, _P, _P, _I64, _I64, _P, _P, _I64, _I, _P]),
    "csa_index_topk_append": (_I, [_P, _P, _P, _P, _I64, _I, _P, _I64, _I, _I, _I, _I, _I, _I, _P, _P, _P, _SZ,
                                   _P, _P, _P, _P, _P, _I, _I, _I, _I, _I, _P, _F, _F, _I64, _P, _SZ, _I, _P, _P,
                                   _I64, _I64, _P, _P, _I64, _I64, _P, _P, _I64, _I, _P]),
    "lcs_attend_workspace": (_SZ, [_I, _I, _I, _I64]),
    "csa_attend": (_I, [_P, _P, _P, _I64, _P, _I, _P, _I64, _I64, _I, _P, _P, _I64, _I, _I, _I, _I, _F, _F, _F,
                        _P, _P, _SZ, _P]),
    "hca_attend": (_I, [_P, _P, _P, _I64, _I64, _I, _P, _I64, _I64, _I, _P, _P, _I64, _I, _I, _I, _I, _F, _F,
                        _F, _P, _P, _SZ, _P]),
    "grouped_out_proj_workspace": (_SZ, [_I, _I, _I]),
    "grouped_out_proj": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "grouped_out_proj_residual": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P, _SZ, _P]),
    "grouped_out_proj_noalloc_max_bytes": (_SZ, []),
    "grouped_out_proj_noalloc": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _I, _P, _P]),
    "input_proj": (_I, [_P, _I, _I, _P, _I, _I, _P, _P, _P, _P, _P]),
    "lcs_timing_enable": (_I, [_I]),
    "lcs_timing_read": (_I, [ctypes.c_char_p, ctypes.POINTER(ctypes.c_double), ctypes.POINTER(ctypes.c_int64)]),
}

_lib = None


class LcsError(RuntimeError):
    def __init__(self, fn, status):
        msg = lib().lcs_status_string(status).decode() if _lib is not None else str(status)
        super().__init__(f"{fn} failed: {msg} (status {status})")
        self.status = status


def lib():
    """Load liblcs.so once and declare the C signatures; raises if the library is absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is not built; run `python -m long_context_sparse_17_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in SIGNATURES.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


# --------------------------------------------------------------------------------- marshalling
def _ptr(t):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream):
    import torch
    s = torch.cuda.current_stream() if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _check(fn, status):
    if status != LCS_OK:
        raise LcsError(fn, status)


def _bits(t, name):
    """bf16 tensors are passed as their 16-bit patterns; accept bfloat16 or int16/uint16 views."""
    import torch
    if t is None:
        return None
    if t.dtype not in (torch.bfloat16, torch.int16, torch.uint16):
        raise TypeError(f"{name} must be bfloat16")
    return t


def _dt(t, dtype, name):
    if t is not None and t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}")
    return t


def workspace(nbytes, device="cuda", zeroed=False):
    """A device workspace of at least nbytes; zeroed=True zero-fills it (csa_index_topk needs that once,
    before its first call; every call leaves it ready for the next)."""
    import torch
    alloc = torch.zeros if zeroed else torch.empty
    return alloc(max(int(nbytes), 256), dtype=torch.uint8, device=device)


# --------------------------------------------------------------------------------- entry points
def csa_compress_kv(kv_tok, kv_score, ik_tok, ik_score, *, tok0, blk_begin, n_blk, m, overlap, gamma_kv,
                    kv_out, ring_cap=0, ik_out=None, ik_scale=None, ik_fp8=True, eps=1e-6,
                    rope_theta=10000.0, rope_offset=0, stream=None):
    """kv_tok [B,T,512] bf16, kv_score [B,T] f32, ik_tok [B,T,dI] bf16 | None, kv_out [B,kv_ld,512]."""
    import torch
    B, T, c = kv_tok.shape
    _bits(kv_tok, "kv_tok"); _bits(gamma_kv, "gamma_kv"); _bits(kv_out, "kv_out")
    _dt(kv_score, torch.float32, "kv_score"); _dt(ik_score, torch.float32, "ik_score")
    dI = ik_tok.shape[-1] if ik_tok is not None else 0
    ik_ld = ik_out.shape[1] if ik_out is not None else 0
    st = lib().csa_compress_kv(_ptr(kv_tok), _ptr(kv_score), _ptr(ik_tok), _ptr(ik_score), B, T, tok0, blk_begin,
                               n_blk, m, overlap, c, dI, _ptr(gamma_kv), eps, rope_theta, rope_offset,
                               _ptr(kv_out), kv_out.shape[1], ring_cap, _ptr(ik_out), _ptr(ik_scale), ik_ld,
                               LCS_IK_FP8 if ik_fp8 else LCS_IK_BF16, _stream(stream))
    _check("csa_compress_kv", st)


def hca_compress_kv(kv_tok, kv_score, *, tok0, blk_begin, n_blk, m, gamma_kv, kv_out, ring_cap=0, eps=1e-6,
                    rope_theta=10000.0, rope_offset=0, stream=None):
    """HCA compression (m = 128) or the window fill (m = 1, ring_cap = ring size)."""
    import torch
    B, T, c = kv_tok.shape
    _bits(kv_tok, "kv_tok"); _dt(kv_score, torch.float32, "kv_score")
    st = lib().hca_compress_kv(_ptr(kv_tok), _ptr(kv_score), B, T, tok0, blk_begin, n_blk, m, c, _ptr(gamma_kv),
                               eps, rope_theta, rope_offset, _ptr(kv_out), kv_out.shape[1], ring_cap,
                               _stream(stream))
    _check("hca_compress_kv", st)


def kv_decode_state_bytes(B):
    return lib().kv_decode_state_bytes(B)


def _append_argv(kv_tok, kv_score, ik_tok, ik_score, pos, *, m, overlap, gamma_kv, state, kv_out, kv_ring=0,
                 win=None, ring_cap=0, ik_out=None, ik_scale=None, ik_fp8=True, eps=1e-6, rope_theta=10000.0,
                 rope_offset=0, kv_scale=None, win_scale=None):
    """The C arguments of kv_decode_append (without the stream)."""
    import torch
    B, c = kv_tok.shape
    kv8 = kv_out.dtype == torch.uint8
    _bits(kv_tok, "kv_tok"); _bits(gamma_kv, "gamma_kv")
    if not kv8:
        _bits(kv_out, "kv_out"); _bits(win, "win")
    elif win is not None and win.dtype != torch.uint8:
        raise TypeError("fp8 K=V: win must hold uint8 codes like kv_out")
    _dt(kv_score, torch.float32, "kv_score"); _dt(ik_score, torch.float32, "ik_score"); _dt(pos, torch.int64, "pos")
    dI = ik_tok.shape[-1] if ik_tok is not None else 0
    ik_ld = ik_out.shape[1] if ik_out is not None else 0
    return (_ptr(kv_tok), _ptr(kv_score), _ptr(ik_tok), _ptr(ik_score), _ptr(pos), B, m, overlap, c, dI,
            _ptr(gamma_kv), eps, rope_theta, rope_offset, _ptr(state), state.numel() * state.element_size(),
            LCS_KV_FP8 if kv8 else LCS_KV_BF16, _ptr(win), _ptr(win_scale), win.shape[1] if win is not None else 0,
            ring_cap, _ptr(kv_out), _ptr(kv_scale), kv_out.shape[1], kv_ring, _ptr(ik_out), _ptr(ik_scale), ik_ld,
            LCS_IK_FP8 if ik_fp8 else LCS_IK_BF16)


def kv_decode_append(kv_tok, kv_score, ik_tok, ik_score, pos, *, stream=None, **kw):
    """Append token pos[b] of every sequence b (pos < 0: skip).  kv_tok [B,512] bf16, kv_score [B] f32,
    ik_tok [B,dI] bf16 | None, pos [B] int64, state: uint8 buffer of kv_decode_state_bytes(B) bytes.
    kv_out / win bf16, or uint8 E4M3FN codes with kv_scale / win_scale [B, ld] f32 (fp8 K=V).
    Keywords: m, overlap, gamma_kv, state, kv_out (required); kv_ring, win, ring_cap, ik_out, ik_scale,
    ik_fp8, eps, rope_theta, rope_offset, kv_scale, win_scale."""
    argv = _append_argv(kv_tok, kv_score, ik_tok, ik_score, pos, **kw)
    _check("kv_decode_append", lib().kv_decode_append(*argv, _stream(stream)))


def kv_quantize_fp8(kv, *, codes, scales, stream=None):
    """kv [..., 512] bf16 rows -> codes [..., 512] uint8 (E4M3FN) and scales [...] f32 (absmax / 448)."""
    import torch
    _bits(kv, "kv"); _dt(codes, torch.uint8, "codes"); _dt(scales, torch.float32, "scales")
    rows = kv.numel() // 512
    if codes.numel() != rows * 512 or scales.numel() != rows:
        raise ValueError("codes / scales do not match kv")
    _check("kv_quantize_fp8", lib().kv_quantize_fp8(_ptr(kv), rows, _ptr(codes), _ptr(scales), _stream(stream)))


def mhc_sinkhorn(logits, *, iters=20, out, stream=None):
    """logits [T, n, n] f32 -> out [T, n, n] f32 (doubly stochastic after Sinkhorn-Knopp)."""
    import torch
    T, n, n2 = logits.shape
    if n != n2:
        raise ValueError("logits must be [T, n, n]")
    _dt(logits, torch.float32, "logits"); _dt(out, torch.float32, "out")
    _check("mhc_sinkhorn", lib().mhc_sinkhorn(_ptr(logits), T, n, iters, _ptr(out), _stream(stream)))


def mhc_mix(x, y, logits, *, iters=20, x_out, h_out=None, stream=None):
    """x [T, n, d] bf16 streams, y [T, d] bf16 layer output, logits [T, n*n + 2n] f32 -> x_out, h_out."""
    import torch
    T, n, d = x.shape
    _bits(x, "x"); _bits(y, "y"); _bits(x_out, "x_out"); _bits(h_out, "h_out")
    _dt(logits, torch.float32, "logits")
    if logits.shape != (T, n * n + 2 * n):
        raise ValueError("logits must be [T, n*n + 2n]")
    _check("mhc_mix", lib().mhc_mix(_ptr(x), _ptr(y), _ptr(logits), T, n, d, iters, _ptr(x_out), _ptr(h_out),
                                     _stream(stream)))


def csa_index_topk_workspace(B, Tq, n_cap, k):
    return lib().csa_index_topk_workspace(B, Tq, n_cap, k)


def _index_argv(q_idx, w_idx, ik_cache, ik_scale, q_pos, *, n_cap, m, k, topk_idx, topk_score=None, ws=None):
    """The C arguments of csa_index_topk (without the stream) and the workspace they reference."""
    import torch
    B, Tq, H_I, dI = q_idx.shape
    fp8 = ik_cache.dtype == torch.uint8
    _dt(q_pos, torch.int64, "q_pos"); _dt(topk_idx, torch.int32, "topk_idx")
    if ws is None:
        ws = workspace(csa_index_topk_workspace(B, Tq, n_cap, k), q_idx.device, zeroed=True)
    return (_ptr(q_idx), _ptr(w_idx), _ptr(ik_cache), _ptr(ik_scale), ik_cache.shape[1],
            LCS_IK_FP8 if fp8 else LCS_IK_BF16, _ptr(q_pos), n_cap, B, Tq, H_I, dI, m, k, _ptr(topk_idx),
            _ptr(topk_score), _ptr(ws), ws.numel()), ws


def csa_index_topk(q_idx, w_idx, ik_cache, ik_scale, q_pos, *, n_cap, m, k, topk_idx, topk_score=None,
                   ws=None, stream=None):
    """q_idx [B,Tq,H_I,dI] bf16, w_idx [B,Tq,H_I] bf16, ik_cache [B,ik_ld,dI] uint8 (fp8) or bf16.
    ws: a workspace(csa_index_topk_workspace(...), zeroed=True), reusable across calls (see lcs.h)."""
    argv, ws = _index_argv(q_idx, w_idx, ik_cache, ik_scale, q_pos, n_cap=n_cap, m=m, k=k, topk_idx=topk_idx,
                           topk_score=topk_score, ws=ws)
    _check("csa_index_topk", lib().csa_index_topk(*argv, _stream(stream)))


def hca_attend_append(q, gamma_q, sink, q_pos, *, n_cap, window, out, append, scale=None, eps=1e-6,
                      rope_theta=10000.0, rope_offset=0, ws=None, stream=None):
    """An HCA decode step's token append and attention in one call.  q [B,1,H,512] bf16 raw; `append`: a dict
    of kv_decode_append's arguments (kv_tok, kv_score, ik_tok, ik_score, pos and its keywords); the
    attention reads the cache (kv_out, kv_scale) and ring (win, win_scale) the append writes."""
    B, Tq, H, c = q.shape
    scale = 1.0 / (c ** 0.5) if scale is None else scale
    if ws is None:
        ws = workspace(attend_workspace(B, Tq, H, n_cap + window), q.device)
    ap = dict(append)
    aargv = _append_argv(ap.pop("kv_tok"), ap.pop("kv_score"), ap.pop("ik_tok"), ap.pop("ik_score"), ap.pop("pos"),
                         **ap)
    st = lib().hca_attend_append(_ptr(q), _ptr(gamma_q), n_cap, window, _ptr(sink), _ptr(q_pos), rope_offset, B, Tq,
                                 H, c, scale, eps, rope_theta, _ptr(out), _ptr(ws), ws.numel(), *aargv,
                                 _stream(stream))
    _check("hca_attend_append", st)


def csa_index_topk_append(q_idx, w_idx, ik_cache, ik_scale, q_pos, *, n_cap, m, k, topk_idx, append,
                          topk_score=None, ws=None, stream=None):
    """csa_index_topk, and in the same call the decode token append described by `append`: a dict of
    kv_decode_append's arguments (kv_tok, kv_score, ik_tok, ik_score, pos and its keywords)."""
    argv, ws = _index_argv(q_idx, w_idx, ik_cache, ik_scale, q_pos, n_cap=n_cap, m=m, k=k, topk_idx=topk_idx,
                           topk_score=topk_score, ws=ws)
    ap = dict(append)
    aargv = _append_argv(ap.pop("kv_tok"), ap.pop("kv_score"), ap.pop("ik_tok"), ap.pop("ik_score"), ap.pop("pos"),
                         **ap)
    _check("csa_index_topk_append", lib().csa_index_topk_append(*argv, *aargv, _stream(stream)))


def attend_workspace(B, Tq, H, max_keys):
    return lib().lcs_attend_workspace(B, Tq, H, max_keys)


def csa_attend(q, gamma_q, kv_cache, topk_idx, win_ring, sink, q_pos, *, window, ring_cap, out, scale=None,
               eps=1e-6, rope_theta=10000.0, rope_offset=0, ws=None, kv_scale=None, win_scale=None, stream=None):
    """q [B,Tq,H,512] bf16 raw; kv_cache [B,kv_ld,512]; topk_idx [B,Tq,k] int32; win_ring [B,win_ld,512].
    kv_cache / win_ring bf16, or uint8 E4M3FN codes with kv_scale / win_scale [B, ld] f32 (fp8 K=V)."""
    import torch
    B, Tq, H, c = q.shape
    k = topk_idx.shape[-1]
    scale = 1.0 / (c ** 0.5) if scale is None else scale
    if ws is None:
        ws = workspace(attend_workspace(B, Tq, H, k + window), q.device)
    if kv_cache.dtype == torch.uint8:
        st = lib().csa_attend_kv8(_ptr(q), _ptr(gamma_q), _ptr(kv_cache), _ptr(kv_scale), kv_cache.shape[1],
                                  _ptr(topk_idx), k, _ptr(win_ring), _ptr(win_scale),
                                  win_ring.shape[1] if win_ring is not None else 0, ring_cap, window, _ptr(sink),
                                  _ptr(q_pos), rope_offset, B, Tq, H, c, scale, eps, rope_theta, _ptr(out), _ptr(ws),
                                  ws.numel(), _stream(stream))
        _check("csa_attend_kv8", st)
        return
    st = lib().csa_attend(_ptr(q), _ptr(gamma_q), _ptr(kv_cache), kv_cache.shape[1], _ptr(topk_idx), k,
                          _ptr(win_ring), win_ring.shape[1] if win_ring is not None else 0, ring_cap, window,
                          _ptr(sink), _ptr(q_pos), rope_offset, B, Tq, H, c, scale, eps, rope_theta, _ptr(out),
                          _ptr(ws), ws.numel(), _stream(stream))
    _check("csa_attend", st)


def hca_attend(q, gamma_q, kv_cache, win_ring, sink, q_pos, *, n_cap, m, window, ring_cap, out, scale=None,
               eps=1e-6, rope_theta=10000.0, rope_offset=0, ws=None, kv_scale=None, win_scale=None, stream=None):
    """Dense attention over entries 0 .. min(t/m, n_cap)-1 plus the window (bf16 or fp8 K=V, as csa_attend)."""
    import torch
    B, Tq, H, c = q.shape
    scale = 1.0 / (c ** 0.5) if scale is None else scale
    if ws is None:
        ws = workspace(attend_workspace(B, Tq, H, n_cap + window), q.device)
    if kv_cache.dtype == torch.uint8:
        st = lib().hca_attend_kv8(_ptr(q), _ptr(gamma_q), _ptr(kv_cache), _ptr(kv_scale), kv_cache.shape[1], n_cap, m,
                                  _ptr(win_ring), _ptr(win_scale), win_ring.shape[1] if win_ring is not None else 0,
                                  ring_cap, window, _ptr(sink), _ptr(q_pos), rope_offset, B, Tq, H, c, scale, eps,
                                  rope_theta, _ptr(out), _ptr(ws), ws.numel(), _stream(stream))
        _check("hca_attend_kv8", st)
        return
    st = lib().hca_attend(_ptr(q), _ptr(gamma_q), _ptr(kv_cache), kv_cache.shape[1], n_cap, m, _ptr(win_ring),
                          win_ring.shape[1] if win_ring is not None else 0, ring_cap, window, _ptr(sink),
                          _ptr(q_pos), rope_offset, B, Tq, H, c, scale, eps, rope_theta, _ptr(out), _ptr(ws),
                          ws.numel(), _stream(stream))
    _check("hca_attend", st)


def grouped_out_proj_workspace(M, g, d_g):
    return lib().grouped_out_proj_workspace(M, g, d_g)


def grouped_out_proj(o, w_g, w_o, *, H, y, ws=None, stream=None):
    """o [M, H*512] bf16; w_g [g, d_g, (H/g)*512]; w_o [d, g*d_g]; y [M, d]."""
    M = o.shape[0]
    g, d_g, _ = w_g.shape
    d = w_o.shape[0]
    if ws is None:
        ws = workspace(grouped_out_proj_workspace(M, g, d_g), o.device)
    st = lib().grouped_out_proj(_ptr(o), _ptr(w_g), _ptr(w_o), M, H, HEAD_DIM, g, d_g, d, _ptr(y), _ptr(ws),
                                ws.numel(), _stream(stream))
    _check("grouped_out_proj", st)


def grouped_out_proj_residual(o, w_g, w_o, resid, *, H, y, ws=None, stream=None):
    """y = grouped projection of o + resid ([M, d] bf16; resid may be y)."""
    M = o.shape[0]
    g, d_g, _ = w_g.shape
    d = w_o.shape[0]
    _bits(resid, "resid")
    if ws is None:
        ws = workspace(grouped_out_proj_workspace(M, g, d_g), o.device)
    st = lib().grouped_out_proj_residual(_ptr(o), _ptr(w_g), _ptr(w_o), _ptr(resid), M, H, HEAD_DIM, g, d_g, d,
                                         _ptr(y), _ptr(ws), ws.numel(), _stream(stream))
    _check("grouped_out_proj_residual", st)


def grouped_out_proj_noalloc(o, w_g, w_o, *, H, y, stream=None):
    """grouped_out_proj without a workspace: z in the library's static device scratch (see lcs.h)."""
    M = o.shape[0]
    g, d_g, _ = w_g.shape
    d = w_o.shape[0]
    st = lib().grouped_out_proj_noalloc(_ptr(o), _ptr(w_g), _ptr(w_o), M, H, HEAD_DIM, g, d_g, d, _ptr(y),
                                        _stream(stream))
    _check("grouped_out_proj_noalloc", st)


def input_proj(h, w_in, segments, *, stream=None):
    """h [M, d] bf16, w_in [n_rows, d] bf16 (output-major, n_rows % 16 == 0); segments: list of
    (width, dst tensor) in column order; dst is [M, >= width] (row stride = dst.stride(0)) bf16 or f32,
    or 1-D [M] for width 1."""
    import torch
    M, d = h.shape
    _bits(h, "h"); _bits(w_in, "w_in")
    n = len(segments)
    widths = (ctypes.c_int * n)(*[int(wd) for wd, _ in segments])
    dsts = (ctypes.c_void_p * n)(*[t.data_ptr() for _, t in segments])
    lds = (ctypes.c_int64 * n)(*[(t.stride(0) if t.dim() > 1 else 1) for _, t in segments])
    f32 = (ctypes.c_int * n)(*[int(t.dtype == torch.float32) for _, t in segments])
    for wd, t in segments:
        if not t.is_cuda or t.dtype not in (torch.float32, torch.bfloat16):
            raise TypeError("segment destinations must be bf16 or f32 GPU tensors")
        if (t.dim() > 1 and t.stride(-1) != 1) or t.shape[0] != M:
            raise ValueError("segment destination must be [M, >= width] with unit column stride")
    st = lib().input_proj(_ptr(h), M, d, _ptr(w_in), w_in.shape[0], n, widths, dsts, lds, f32, _stream(stream))
    _check("input_proj", st)


def timing_enable(on=True):
    _check("lcs_timing_enable", lib().lcs_timing_enable(1 if on else 0))


def timing_read(name):
    """(total milliseconds, launches) of the library's kernels whose name contains `name`."""
    ms = ctypes.c_double(0.0)
    n = ctypes.c_int64(0)
    _check("lcs_timing_read", lib().lcs_timing_read(name.encode(), ctypes.byref(ms), ctypes.byref(n)))
    return ms.value, n.value
