"""End-to-end small layers: raw seeded per-token inputs -> GPU chain (compress, window fill, indexer +
top-k, attention, grouped projection) and the oracle's chain on the same raw inputs.

Used by the end-to-end GPU tests and by __graft_entry__.smoke().
"""
from __future__ import annotations

import math

import numpy as np
import torch

import long_context_sparse_17_amd as L
import oracle as O
import synth
from lcs_testutil import errors, from_bits, to_np_bf16

DEV = "cuda"
RING = 256


def _f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def _raw(B, T1, H, H_I, dI, cfg):
    s = 1.28
    return dict(
        kv=synth.normal_bf16((B, T1, 512), s, cfg, 1), ks=synth.normal_f32((B, T1), s, cfg, 2),
        ik=synth.normal_bf16((B, T1, dI), s, cfg, 3), iks=synth.normal_f32((B, T1), s, cfg, 4),
        q=synth.normal_bf16((B, 1, H, 512), s, cfg, 5), qi=synth.normal_bf16((B, 1, H_I, dI), s, cfg, 6),
        wi=synth.normal_bf16((B, 1, H_I), s, cfg, 7), sink=synth.normal_f32((H,), 1.0, cfg, 8),
        wg=synth.normal_bf16((8, 64, H * 512 // 8), 0.02, cfg, 9), wo=synth.normal_bf16((96, 8 * 64), 0.02, cfg, 10))


def _window_fill(r, B, t, W, rope_offset):
    ring = torch.zeros((B, RING, 512), dtype=torch.bfloat16, device=DEV)
    w0 = max(0, t - W + 1)
    g = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    L.hca_compress_kv(from_bits(r["kv"][:, w0:t + 1]), _f32(r["ks"][:, w0:t + 1]), tok0=w0, blk_begin=w0,
                      n_blk=t + 1 - w0, m=1, gamma_kv=g, kv_out=ring, ring_cap=RING, rope_offset=rope_offset)
    return ring


def run_csa(B=2, t=600, H=64, H_I=64, dI=128, k=64, W=128, cfg=700, rope_offset=0, fp8=True):
    """One CSA decode query at token t per sequence.  Returns dict of GPU and oracle results."""
    r = _raw(B, t + 1, H, H_I, dI, cfg)
    m, ov = 4, 4
    n_cap = t // m
    g = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    kv_cache = torch.zeros((B, n_cap, 512), dtype=torch.bfloat16, device=DEV)
    ik_cache = torch.zeros((B, n_cap, dI), dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
    ik_sc = torch.zeros((B, n_cap), dtype=torch.float32, device=DEV)
    L.csa_compress_kv(from_bits(r["kv"]), _f32(r["ks"]), from_bits(r["ik"]), _f32(r["iks"]), tok0=0, blk_begin=0,
                      n_blk=n_cap, m=m, overlap=ov, gamma_kv=g, kv_out=kv_cache, ik_out=ik_cache,
                      ik_scale=ik_sc if fp8 else None, ik_fp8=fp8, rope_offset=rope_offset)
    ring = _window_fill(r, B, t, W, rope_offset)
    pos = torch.full((B, 1), t, dtype=torch.int64, device=DEV)
    topk = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(from_bits(r["qi"]), from_bits(r["wi"]), ik_cache, ik_sc if fp8 else None, pos, n_cap=n_cap,
                     m=m, k=k, topk_idx=topk)
    o = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
    L.csa_attend(from_bits(r["q"]), g, kv_cache, topk, ring, _f32(r["sink"]), pos, window=W, ring_cap=RING, out=o,
                 rope_offset=rope_offset)
    y = torch.empty((B, 96), dtype=torch.bfloat16, device=DEV)
    L.grouped_out_proj(o.view(B, H * 512), from_bits(r["wg"]), from_bits(r["wo"]), H=H, y=y)
    torch.cuda.synchronize()
    res = dict(gpu_topk=topk.cpu().numpy()[:, 0], gpu_o=to_np_bf16(o)[:, 0], gpu_y=to_np_bf16(y), ref_o=[],
               ref_sel=[], ref_scores=[], ref_o_on_gpu_set=[], ref_o_exact_indexer=[], ref_y=None)
    ones = np.ones(512)
    for b in range(B):
        f = lambda a: synth.bf16_bits_to_f64(a)  # noqa: E731
        args = (f(r["kv"][b]), r["ks"][b].astype(np.float64), f(r["ik"][b]), r["iks"][b].astype(np.float64),
                f(r["q"][b]), f(r["qi"][b]), f(r["wi"][b]), r["sink"].astype(np.float64), [t])
        kw = dict(m=m, ov=ov, W=W, k=k, fp8=fp8, rope_offset=rope_offset)
        o_ref, sel, sc = O.csa_layer(*args, **kw)
        res["ref_o"].append(o_ref[0])
        res["ref_sel"].append(sel[0])
        res["ref_scores"].append(sc[0])
        if fp8:
            o_ex, sel_ex, _ = O.csa_layer(*args, **dict(kw, fp8=False))
            res["ref_o_exact_indexer"].append(o_ex[0])
            res.setdefault("ref_sel_exact", []).append(sel_ex[0])
        # oracle attention on the GPU's selection (used where the sets differ inside the tie band)
        ent = O.compress_kv(args[0], args[1], m, ov, ones, 1e-6, 10000.0, rope_offset)
        win = O.window_entries(args[0], ones, 1e-6, 10000.0, rope_offset)
        res["ref_o_on_gpu_set"].append(O.csa_attend_one(args[4][0], ones, ent, res["gpu_topk"][b], win, args[7], t,
                                                        W, 1 / math.sqrt(512), 1e-6, 10000.0, rope_offset))
    res["ref_o"] = np.stack(res["ref_o"])
    res["ref_o_on_gpu_set"] = np.stack(res["ref_o_on_gpu_set"])
    _, res["ref_y"] = O.grouped_out_proj(res["ref_o"].reshape(B, H * 512), f(r["wg"]), f(r["wo"]))
    return res


def run_hca(B=2, t=677, H=64, W=128, m=128, cfg=710, rope_offset=0, sink_inf=False):
    r = _raw(B, t + 1, H, 8, 64, cfg)
    if sink_inf:
        r["sink"] = np.full(H, -np.inf, np.float32)
    n_cap = t // m
    g = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    kv_cache = torch.zeros((B, max(n_cap, 1), 512), dtype=torch.bfloat16, device=DEV)
    if n_cap:
        L.hca_compress_kv(from_bits(r["kv"]), _f32(r["ks"]), tok0=0, blk_begin=0, n_blk=n_cap, m=m, gamma_kv=g,
                          kv_out=kv_cache, rope_offset=rope_offset)
    ring = _window_fill(r, B, t, W, rope_offset)
    pos = torch.full((B, 1), t, dtype=torch.int64, device=DEV)
    o = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
    L.hca_attend(from_bits(r["q"]), g, kv_cache, ring, _f32(r["sink"]), pos, n_cap=n_cap, m=m, window=W,
                 ring_cap=RING, out=o, rope_offset=rope_offset)
    torch.cuda.synchronize()
    ref = []
    for b in range(B):
        f = lambda a: synth.bf16_bits_to_f64(a)  # noqa: E731
        ref.append(O.hca_layer(f(r["kv"][b]), r["ks"][b].astype(np.float64), f(r["q"][b]),
                               r["sink"].astype(np.float64), [t], m=m, W=W, rope_offset=rope_offset)[0])
    return dict(gpu_o=to_np_bf16(o)[:, 0], ref_o=np.stack(ref))


def csa_report(res, k):
    """Errors of a run_csa result; the attention comparison uses the oracle on the GPU's selection
    only where the GPU and oracle sets differ inside the tie band of the oracle's scores."""
    out = {"topk_mismatch_rows": 0}
    B = res["gpu_o"].shape[0]
    ref_o = res["ref_o"].copy()
    for b in range(B):
        gsel = res["gpu_topk"][b]
        rsel = res["ref_sel"][b]
        if not np.array_equal(gsel, rsel):
            sc = res["ref_scores"][b]
            n = sc.shape[0]
            kth = sc[np.lexsort((np.arange(n), -sc))[min(k, n) - 1]]
            diff = np.setxor1d(gsel[gsel >= 0], rsel[rsel >= 0])
            band = 1e-3 * max(1.0, abs(kth))         # fp8 keys quantised from fp32 vs fp64 pooled values
            assert np.all(np.abs(sc[diff] - kth) <= band), "top-k differs outside the tie band"
            out["topk_mismatch_rows"] += 1
            ref_o[b] = res["ref_o_on_gpu_set"][b]
    out["o"] = errors(res["gpu_o"], ref_o)
    out["y"] = errors(res["gpu_y"], res["ref_y"])
    if res["ref_o_exact_indexer"]:
        ex = np.stack(res["ref_o_exact_indexer"])
        out["o_vs_exact_indexer"] = errors(res["gpu_o"], ex)
        out["oracle_fp8_vs_exact"] = errors(res["ref_o"], ex)
        ov = []
        for b in range(B):
            a, e = res["gpu_topk"][b], res["ref_sel_exact"][b]
            a, e = a[a >= 0], e[e >= 0]
            ov.append(np.intersect1d(a, e).size / max(1, e.size))
        out["selection_overlap_vs_exact"] = float(min(ov))
    return out
