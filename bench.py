"""Benchmark: CSA+HCA attention decode at 1M context on one MI355X.

Workload: the hybrid 4-layer decode stack (CSA, HCA, CSA, HCA), batch 8, context 2^20 tokens, 64 heads
of dim 512, window 128, sink, CSA top-k 1024 with a 64x128 fp8 indexer, HCA m' = 128, grouped output
projection g = 8 -> d_g = 1024 -> d = 4096.  One step = one decode token for every sequence through
all four layers: window fill, block compression, indexer + top-k (CSA), attention, projection.
Inputs are synthetic and resident in HBM before timing; the caches are built by the library's own
compression kernels from seeded per-token data (untimed).

Prints one JSON line: tokens/s/layer = B * layers / step time, with the HBM roofline of the dominant
kernel (timed with HIP events on its launch stream by the library) and the CPU oracle's rate on a
bounded sample of the same workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "CSA+HCA attention decode tokens/s/layer at 1M ctx; % of HBM roofline"
HBM_PEAK_GBS = 8000.0
FP8_PEAK_TFLOPS = 5000.0      # dense fp8 matrix-core peak (published)
BF16_PEAK_TFLOPS = 2500.0     # dense bf16 matrix-core peak (published)


def log(*a):
    print(*a, file=sys.stderr, flush=True)


TRAFFIC_FILE = os.path.join(ROOT, "profiles", "index_score_decode_kernel_hybrid4_decode_1m_traffic.md")


def stored_traffic():
    """HBM bytes per launch of the dominant kernel as measured by the FETCH_SIZE / WRITE_SIZE counter
    passes recorded in profiles/ (copy-calibrated), or None when the kernel source has changed since."""
    import hashlib
    try:
        for line in open(TRAFFIC_FILE):
            if line.strip().startswith("TRAFFIC "):
                rec = json.loads(line.strip()[len("TRAFFIC "):])
                src = open(os.path.join(ROOT, rec["source"]), "rb").read()
                if hashlib.sha256(src).hexdigest() == rec["source_sha256"]:
                    return int(rec["traffic_bytes"])
    except (OSError, ValueError, KeyError):
        pass
    return None


def cpu_baseline(layers, n_seq, min_s=10.0, max_s=30.0):
    """Time the fp64 oracle (as it stands) on n_seq sequences through all layers, inputs copied back
    from the device, repeating the sample until at least min_s seconds of CPU work (at most about
    max_s).  Returns (tokens/s/layer, seconds, threads, sample description)."""
    import numpy as np

    import oracle as O
    import synth
    from long_context_sparse_17_amd.pipeline import RING, CsaDecodeLayer

    def bf(t):
        import torch
        return synth.bf16_bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))

    # host copies (not timed)
    host = []
    for L in layers:
        d = dict(q=bf(L.q[:n_seq, 0]), sink=L.sink.cpu().numpy().astype(np.float64),
                 ring=bf(L.ring[:n_seq]), wg=bf(L.w_g), wo=bf(L.w_o), t=L.t)
        if isinstance(L, CsaDecodeLayer):
            d["csa"] = True
            d["kv"] = [bf(L.kv_cache[b]) for b in range(n_seq)]
            d["kI"] = [O.e4m3_decode(L.ik_cache[b].cpu().numpy()) * L.ik_scale[b].cpu().numpy()[:, None].astype(np.float64)
                       for b in range(n_seq)]
            d["qI"] = bf(L.q_idx[:n_seq, 0])
            d["wI"] = bf(L.w_idx[:n_seq, 0])
            d["k"], d["m"] = L.k, L.m
        else:
            d["csa"] = False
            d["kv"] = [bf(L.kv_cache[b]) for b in range(n_seq)]
            d["m"] = L.m
        host.append(d)
    ones = np.ones(512)

    def unit(b, d):
        """One layer-token: indexer + top-k (CSA), attention, projection."""
        t = d["t"]
        win = np.stack([d["ring"][b][j % RING] for j in range(t - 127, t + 1)])
        n = O.n_visible(t, d["m"])
        if d["csa"]:
            _, _, qI = O.fp8_quantize_rows(d["qI"][b])
            sc = O.index_scores(qI, d["wI"][b], d["kI"][b][:n])
            sel = O.topk_select(sc, d["k"])
            keys = np.concatenate([d["kv"][b][sel[sel >= 0]], win])
        else:
            keys = np.concatenate([d["kv"][b][:n], win])
        o = O.attend_one(d["q"][b], ones, keys, d["sink"], t, 1.0 / np.sqrt(512))
        O.grouped_out_proj(o.reshape(1, -1), d["wg"], d["wo"])

    t0 = time.perf_counter()
    done = 0
    reps = 0
    while True:
        for b in range(n_seq):
            for d in host:
                unit(b, d)
                done += 1
            if time.perf_counter() - t0 > max_s:
                break
        reps += 1
        if time.perf_counter() - t0 >= min_s:
            break
    dt = time.perf_counter() - t0
    # one thread: one CSA and one HCA layer-token of sequence 0 (BLAS limited to a single thread)
    single = None
    try:
        from threadpoolctl import threadpool_limits
        with threadpool_limits(limits=1):
            t1 = time.perf_counter()
            for d in host[:2]:
                unit(0, d)
            ts = time.perf_counter() - t1
        single = {"value": round(2 / ts, 3), "unit": "tokens/s/layer", "cores": 1, "seconds": round(ts, 3),
                  "sample": "sequence 0 through one CSA and one HCA layer (one layer-token each)"}
    except ImportError:
        pass
    threads = int(os.environ.get("OMP_NUM_THREADS", os.cpu_count() or 1))
    try:
        from threadpoolctl import threadpool_info
        nt = [i.get("num_threads") for i in threadpool_info() if i.get("user_api") == "blas"]
        if nt:
            threads = int(max(nt))
    except Exception:
        pass
    return done / dt, dt, threads, f"{n_seq} of {layers[0].B} sequences x {len(layers)} layers, repeated {reps}x " \
                                   f"({done} layer-tokens: indexer + top-k + attention + projection), caches " \
                                   f"copied from the device", single


def fp8_indexer_check(dev, B=2, t=4096, k=256, cfg=900):
    """Part of the oracle leg of the benchmark.  How much the fp8 indexer moves the attention output (the reading that fp8 keys and queries keep
    the method intact): one CSA decode query per sequence at token t, from raw seeded per-token
    vectors.  The GPU path (compression with fp8 indexer keys, window fill, indexer + top-k,
    attention) and the oracle with the fp8 indexer and with an exact one (no quantisation), on the
    same raw inputs.  Reports the rel-L2 distances and the share of the exact top-k the GPU keeps."""
    import numpy as np
    import torch
    import long_context_sparse_17_amd as L
    import oracle as O
    import synth
    H, H_I, dI, W, m, ov, ring = 64, 64, 128, 128, 4, 4, 256
    T1 = t + 1
    s = 1.28
    kv = synth.normal_bf16((B, T1, 512), s, cfg, 1)
    ks = synth.normal_f32((B, T1), s, cfg, 2)
    ik = synth.normal_bf16((B, T1, dI), s, cfg, 3)
    iks = synth.normal_f32((B, T1), s, cfg, 4)
    q = synth.normal_bf16((B, 1, H, 512), s, cfg, 5)
    qi = synth.normal_bf16((B, 1, H_I, dI), s, cfg, 6)
    wi = synth.normal_bf16((B, 1, H_I), s, cfg, 7)
    sink = synth.normal_f32((H,), 1.0, cfg, 8)
    bf = lambda a: torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16).to(dev)  # noqa: E731
    f32 = lambda a: torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(dev)  # noqa: E731
    n_cap = t // m
    g = torch.ones(512, dtype=torch.bfloat16, device=dev)
    kv_cache = torch.zeros((B, n_cap, 512), dtype=torch.bfloat16, device=dev)
    ik_cache = torch.zeros((B, n_cap, dI), dtype=torch.uint8, device=dev)
    ik_sc = torch.zeros((B, n_cap), dtype=torch.float32, device=dev)
    L.csa_compress_kv(bf(kv), f32(ks), bf(ik), f32(iks), tok0=0, blk_begin=0, n_blk=n_cap, m=m, overlap=ov, gamma_kv=g,
                      kv_out=kv_cache, ik_out=ik_cache, ik_scale=ik_sc, ik_fp8=True)
    win = torch.zeros((B, ring, 512), dtype=torch.bfloat16, device=dev)
    w0 = t - W + 1
    L.hca_compress_kv(bf(kv[:, w0:]), f32(ks[:, w0:]), tok0=w0, blk_begin=w0, n_blk=T1 - w0, m=1, gamma_kv=g,
                      kv_out=win, ring_cap=ring)
    pos = torch.full((B, 1), t, dtype=torch.int64, device=dev)
    topk = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    L.csa_index_topk(bf(qi), bf(wi), ik_cache, ik_sc, pos, n_cap=n_cap, m=m, k=k, topk_idx=topk)
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=dev)
    L.csa_attend(bf(q), g, kv_cache, topk, win, f32(sink), pos, window=W, ring_cap=ring, out=out)
    torch.cuda.synchronize()
    got = synth.bf16_bits_to_f64(out.cpu().view(torch.int16).numpy().view(np.uint16))
    gsel = topk.cpu().numpy()
    f = synth.bf16_bits_to_f64
    rl = lambda a, b: float(np.linalg.norm(a - b) / np.linalg.norm(b))  # noqa: E731
    r = {"oracle_fp8_vs_exact": 0.0, "gpu_vs_exact": 0.0, "gpu_vs_oracle_fp8": 0.0, "exact_topk_kept": 1.0}
    for b in range(B):
        args = (f(kv[b]), ks[b].astype(np.float64), f(ik[b]), iks[b].astype(np.float64), f(q[b]), f(qi[b]),
                f(wi[b]), sink.astype(np.float64), [t])
        o8, _, _ = O.csa_layer(*args, m=m, ov=ov, W=W, k=k, fp8=True)
        oe, sel_e, _ = O.csa_layer(*args, m=m, ov=ov, W=W, k=k, fp8=False)
        r["oracle_fp8_vs_exact"] = max(r["oracle_fp8_vs_exact"], rl(o8[0], oe[0]))
        r["gpu_vs_exact"] = max(r["gpu_vs_exact"], rl(got[b, 0], oe[0]))
        r["gpu_vs_oracle_fp8"] = max(r["gpu_vs_oracle_fp8"], rl(got[b, 0], o8[0]))
        se = set(int(x) for x in sel_e[0] if x >= 0)
        sg = set(int(x) for x in gsel[b, 0] if x >= 0)
        r["exact_topk_kept"] = min(r["exact_topk_kept"], len(se & sg) / max(1, len(se)))
    r = {key: round(v, 5) for key, v in r.items()}
    r["what"] = (f"CSA decode, {B} sequences at t = {t} ({n_cap} entries), top-k {k}, raw seeded tokens: rel-L2 of "
                 "the attention output; the oracle with the fp8 indexer against the oracle with an exact one, "
                 "and the GPU against both")
    return r


def _event_time_us(fn, reps, graph=False):
    """Average duration of fn() on the current stream, HIP events around reps back-to-back calls.
    graph=True captures the reps calls into one graph first, so host launch costs do not count."""
    import torch
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    run, n = fn, reps
    if graph:
        s = torch.cuda.Stream()
        s.wait_stream(torch.cuda.current_stream())
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=s):
            for _ in range(reps):
                fn()
        torch.cuda.synchronize()
        run, n = g.replay, 1
        run()
        torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(n):
        run()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) * 1e3 / reps


def mfma_reference(dev):
    """Measured dense bf16 matrix-core ceiling: an 8192^3 GEMM (library kernel) in TFLOP/s."""
    import torch
    n = 8192
    a = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    b = torch.randn(n, n, device=dev, dtype=torch.bfloat16)
    us = _event_time_us(lambda: torch.matmul(a, b), 10)
    return 2.0 * n ** 3 / (us * 1e-6) / 1e12


def decode_append_rows(dev, B):
    """kv_decode_append (one token per sequence, the block ends at this token: pooled-state update,
    window-ring row, entry finished and stored) at batch B, for the CSA layer shape (m = 4, overlap 4,
    fp8 indexer keys of 128 dims) and the HCA shape (m = 128)."""
    import torch
    import long_context_sparse_17_amd as L
    g = torch.Generator(device=dev).manual_seed(5)
    kv = (torch.randn(B, 512, device=dev, generator=g) * 1.28).to(torch.bfloat16)
    ks = torch.randn(B, device=dev, generator=g)
    ik = (torch.randn(B, 128, device=dev, generator=g) * 1.28).to(torch.bfloat16)
    iks = torch.randn(B, device=dev, generator=g)
    gamma = torch.ones(512, device=dev, dtype=torch.bfloat16)
    pos = torch.full((B,), 4095, dtype=torch.int64, device=dev)
    state = torch.zeros(L.kv_decode_state_bytes(B), dtype=torch.uint8, device=dev)
    ring = torch.zeros(B, 256, 512, device=dev, dtype=torch.bfloat16)
    kv_out = torch.zeros(B, 1024, 512, device=dev, dtype=torch.bfloat16)
    ik_out = torch.zeros(B, 1024, 128, device=dev, dtype=torch.uint8)
    ik_sc = torch.zeros(B, 1024, device=dev)
    def prime(t0, **kw):                      # append positions t0 .. 4094: the block ending at 4095 is open
        for t in range(t0, 4095):
            L.kv_decode_append(kv, ks, kw.get("ik"), kw.get("iks"), torch.full((B,), t, dtype=torch.int64, device=dev),
                               **{k: v for k, v in kw.items() if k not in ("ik", "iks")})
    prime(4088, ik=ik, iks=iks, m=4, overlap=4, gamma_kv=gamma, state=state, kv_out=kv_out, win=ring, ring_cap=256,
          ik_out=ik_out, ik_scale=ik_sc)
    csa = _event_time_us(lambda: L.kv_decode_append(kv, ks, ik, iks, pos, m=4, overlap=4, gamma_kv=gamma, state=state,
                                                    kv_out=kv_out, win=ring, ring_cap=256, ik_out=ik_out,
                                                    ik_scale=ik_sc), 200, graph=True)
    state.zero_()
    prime(3968, m=128, overlap=0, gamma_kv=gamma, state=state, kv_out=kv_out, win=ring, ring_cap=256)
    hca = _event_time_us(lambda: L.kv_decode_append(kv, ks, None, None, pos, m=128, overlap=0, gamma_kv=gamma,
                                                    state=state, kv_out=kv_out, win=ring, ring_cap=256), 200,
                         graph=True)
    # bytes per sequence: token (1 KiB + 256 B keys + logits), two state slots read and written, ring row,
    # entry and key written
    slot = (512 + 128 + 8) * 4
    csa_bytes = B * (1024 + 256 + 8 + 2 * 2 * slot + 1024 + 1024 + 128 + 4)
    hca_bytes = B * (1024 + 4 + 2 * (512 + 8) * 4 + 1024 + 1024)
    return {"what": "kv_decode_append: one token per sequence that ends a block (state update, ring row, "
                    "entry + key stored)", "batch": B,
            "csa_us": round(csa, 2), "hca_us": round(hca, 2), "csa_bytes": csa_bytes, "hca_bytes": hca_bytes,
            "bound": "latency (one workgroup per sequence)"}


def mhc_row(dev):
    """mhc_mix on 4096 tokens x 4 streams x 4096 dims, 20 Sinkhorn-Knopp rounds per token: streams
    and the layer output read once, new streams and the next input written once."""
    import torch
    import long_context_sparse_17_amd as L
    T, n, d = 4096, 4, 4096
    g = torch.Generator(device=dev).manual_seed(7)
    x = torch.randn((T, n, d), device=dev, generator=g).to(torch.bfloat16)
    y = torch.randn((T, d), device=dev, generator=g).to(torch.bfloat16)
    lg = torch.randn((T, n * n + 2 * n), device=dev, generator=g)
    xo = torch.empty_like(x)
    h = torch.empty_like(y)
    us = _event_time_us(lambda: L.mhc_mix(x, y, lg, iters=20, x_out=xo, h_out=h), 20)
    nbytes = T * (2 * n * d * 2 + 2 * d * 2 + (n * n + 2 * n) * 4)
    gbs = nbytes / (us * 1e-6) / 1e9
    return {"what": "mhc_mix: T=4096 tokens, n=4 streams, d=4096, 20 rounds", "us": round(us, 2),
            "bytes": nbytes, "achieved_gbs": round(gbs, 1), "bound": "hbm",
            "frac": round(gbs / HBM_PEAK_GBS, 4)}


def prefill_row(dev):
    """CSA chunked prefill at 1M context: 4096 new queries (positions 2^20 - 4096 .. 2^20 - 1) against
    262144 compressed entries (m = 4), fp8 indexer 64 x 128, top-k 1024, 64 query heads, window 128.
    Per-kernel times (HIP events on the launch stream, 3 calls after a warm-up call) and the fp8
    indexer's matrix-core rate: 2 * 64 * 128 flop per visible query-entry pair."""
    import torch
    import long_context_sparse_17_amd as L
    import synth
    N, Tq, n_cap, k, H, H_I, dI, W, ring = 1 << 20, 4096, 1 << 18, 1024, 64, 64, 128, 128, 8192
    codes = synth.device_fp8_codes((1, n_cap, dI), 41)
    scale = (synth.device_normal_f32((1, n_cap), 1.0, 42).abs() + 2.0) / 448.0
    cache = synth.device_normal_bf16((1, n_cap, 512), 1.0, 43)
    win = synth.device_normal_bf16((1, ring, 512), 1.0, 44)
    q = synth.device_normal_bf16((1, Tq, H, 512), 1.0, 45)
    qi = synth.device_normal_bf16((1, Tq, H_I, dI), 1.0, 46)
    wi = synth.device_normal_bf16((1, Tq, H_I), 1.0, 47)
    sink = synth.device_normal_f32((H,), 1.0, 48)
    gq = torch.ones(512, dtype=torch.bfloat16, device=dev)
    pos = torch.arange(N - Tq, N, dtype=torch.int64, device=dev).view(1, Tq)
    topk = torch.empty((1, Tq, k), dtype=torch.int32, device=dev)
    out = torch.empty((1, Tq, H, 512), dtype=torch.bfloat16, device=dev)
    ws_i = L.workspace(L.csa_index_topk_workspace(1, Tq, n_cap, k), zeroed=True)
    ws_a = L.workspace(L.attend_workspace(1, Tq, H, k + W))
    g, d_g, d = 8, 1024, 4096
    w_g = synth.device_normal_bf16((g, d_g, H * 512 // g), 0.02, 49)
    w_o = synth.device_normal_bf16((d, g * d_g), 0.02, 50)
    y = torch.empty((Tq, d), dtype=torch.bfloat16, device=dev)
    ws_p = L.workspace(L.grouped_out_proj_workspace(Tq, g, d_g))

    def call():
        L.csa_index_topk(qi, wi, codes, scale, pos, n_cap=n_cap, m=4, k=k, topk_idx=topk, ws=ws_i)
        L.csa_attend(q, gq, cache, topk, win, sink, pos, window=W, ring_cap=ring, out=out, ws=ws_a)
        L.grouped_out_proj(out.view(Tq, H * 512), w_g, w_o, H=H, y=y, ws=ws_p)

    call()
    torch.cuda.synchronize()
    L.timing_enable(True)
    reps = 3
    for _ in range(reps):
        call()
    torch.cuda.synchronize()
    kern = {}
    for name in ("index_qprep_kernel", "index_score_kernel", "topk_rowwise_kernel", "attend_csa_kernel",
                 "attend_merge_kernel", "out_proj_group_kernel", "out_proj_out_kernel"):
        ms, n = L.timing_read(name)
        if n:
            kern[name] = {"avg_ms": round(ms / n, 4), "launches": n // reps, "per_call_ms": round(ms / reps, 4)}
    L.timing_enable(False)
    pairs = sum((N - Tq + i) // 4 for i in range(Tq))
    flops = 2.0 * pairs * H_I * dI
    # the indexer scores the queries in row batches: its time per call is the sum over its launches
    idx_ms = kern["index_score_kernel"]["per_call_ms"]
    tflops = flops / (idx_ms * 1e-3) / 1e12
    total = sum(v["per_call_ms"] for v in kern.values())
    # attention: 4 * 512 flop per head and key (QK^T and PV), keys = the k selected + the 128-token window
    att_flops = 4.0 * 512 * H * Tq * (k + W)
    att_ms = kern["attend_csa_kernel"]["per_call_ms"]
    # grouped projection: 2 flop per weight and row, both stages
    proj_flops = 2.0 * Tq * (g * d_g * (H * 512 // g) + d * g * d_g)
    proj_ms = kern["out_proj_group_kernel"]["per_call_ms"] + kern["out_proj_out_kernel"]["per_call_ms"]
    del codes, scale, cache, win, q, qi, wi, topk, out, ws_i, ws_a, w_g, w_o, y, ws_p
    torch.cuda.empty_cache()
    return {"what": "CSA chunked prefill, 4096 queries x 262144 entries (1M tokens, m = 4), top-k 1024, 64 heads, "
                    "then the grouped output projection of the 4096 rows (8 x 1024 -> 4096)",
            "ms_per_call": round(total, 3), "kernels": kern, "indexer_flops": flops,
            "indexer_ms": round(idx_ms, 4), "indexer_tflops": round(tflops, 1), "indexer_bound": "mfma (fp8)", "fp8_peak_tflops": FP8_PEAK_TFLOPS,
            "indexer_frac": round(tflops / FP8_PEAK_TFLOPS, 4),
            "attention_tflops": round(att_flops / (att_ms * 1e-3) / 1e12, 1),
            "attention_frac": round(att_flops / (att_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4),
            "out_proj_ms": round(proj_ms, 4), "out_proj_tflops": round(proj_flops / (proj_ms * 1e-3) / 1e12, 1),
            "out_proj_frac": round(proj_flops / (proj_ms * 1e-3) / 1e12 / BF16_PEAK_TFLOPS, 4)}


def _graph_time_ms(fn, n_sets, reps=40):
    """Average time of fn(i) over reps calls captured into one graph (input set i % n_sets), after warm-up."""
    import torch
    for i in range(3):
        fn(i)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        for i in range(reps):
            fn(i)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    g.replay()
    e1.record()
    torch.cuda.synchronize()
    return e0.elapsed_time(e1) / reps


def hca_decode_64k_row(dev, n_sets=20):
    """HCA decode at 64K context: 64 sequences, 512 visible entries each + the 128-token window, 64 heads,
    sink.  One step = hca_attend for every sequence.  20 input sets (cache, ring, queries) rotate so that
    the Infinity Cache does not serve repeats.  Bytes: every visible entry and window row once (1 KiB),
    q read and o written once."""
    import torch
    import long_context_sparse_17_amd as L
    import synth
    B, n_cap, H, W, ring, t = 64, 512, 64, 128, 256, 65536
    sets = [(synth.device_normal_bf16((B, n_cap, 512), 1.0, 3_000_000 + 10 * i),
             synth.device_normal_bf16((B, ring, 512), 1.0, 3_000_001 + 10 * i),
             synth.device_normal_bf16((B, 1, H, 512), 1.28, 3_000_002 + 10 * i)) for i in range(n_sets)]
    sink = synth.device_normal_f32((H,), 1.0, 3_000_003)
    gq = torch.ones(512, dtype=torch.bfloat16, device=dev)
    pos = torch.full((B, 1), t, dtype=torch.int64, device=dev)
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=dev)
    ws = L.workspace(L.attend_workspace(B, 1, H, n_cap + W))

    def fn(i):
        cache, win, q = sets[i % n_sets]
        L.hca_attend(q, gq, cache, win, sink, pos, n_cap=n_cap, m=128, window=W, ring_cap=ring, out=out, ws=ws)

    ms = _graph_time_ms(fn, n_sets)
    nbytes = B * (n_cap + W) * 1024 + B * H * 512 * 2 * 2
    gbs = nbytes / (ms * 1e-3) / 1e9
    del sets, out, ws
    torch.cuda.empty_cache()
    return {"what": "HCA decode, 64 sequences at 64K context (512 entries + 128-token window), 64 heads",
            "ms_per_step": round(ms, 4), "tokens_per_s_per_layer": round(B / (ms * 1e-3), 1),
            "input_sets": n_sets, "roofline": {"bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
                                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                               "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def csa_decode_128k_row(dev, n_sets=7):
    """CSA decode at 128K context (the Flash configuration): 32 sequences, 32768 compressed entries each,
    fp8 indexer 64 x 128, top-k 512, 64 heads, window 128.  One step = csa_index_topk + csa_attend.
    7 input sets (caches, keys, queries) rotate.  Bytes: every visible indexer key and scale once (132 B),
    each selected entry and window row once (1 KiB), the queries, head weights, q and o once."""
    import torch
    import long_context_sparse_17_amd as L
    import synth
    B, n_cap, H, H_I, dI, k, W, ring, t = 32, 32768, 64, 64, 128, 512, 128, 256, 131072
    sets = []
    for i in range(n_sets):
        base = 4_000_000 + 100 * i
        sets.append(dict(codes=synth.device_fp8_codes((B, n_cap, dI), base + 1),
                         scale=(synth.device_normal_f32((B, n_cap), 1.0, base + 2).abs() + 2.0) / 448.0,
                         cache=synth.device_normal_bf16((B, n_cap, 512), 1.0, base + 3),
                         win=synth.device_normal_bf16((B, ring, 512), 1.0, base + 4),
                         q=synth.device_normal_bf16((B, 1, H, 512), 1.28, base + 5),
                         qi=synth.device_normal_bf16((B, 1, H_I, dI), 1.28, base + 6),
                         wi=synth.device_normal_bf16((B, 1, H_I), 1.28, base + 7)))
    sink = synth.device_normal_f32((H,), 1.0, 4_000_099)
    gq = torch.ones(512, dtype=torch.bfloat16, device=dev)
    pos = torch.full((B, 1), t, dtype=torch.int64, device=dev)
    topk = torch.empty((B, 1, k), dtype=torch.int32, device=dev)
    out = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=dev)
    ws_i = L.workspace(L.csa_index_topk_workspace(B, 1, n_cap, k), zeroed=True)
    ws_a = L.workspace(L.attend_workspace(B, 1, H, k + W))

    def fn(i):
        d = sets[i % n_sets]
        L.csa_index_topk(d["qi"], d["wi"], d["codes"], d["scale"], pos, n_cap=n_cap, m=4, k=k, topk_idx=topk,
                         ws=ws_i)
        L.csa_attend(d["q"], gq, d["cache"], topk, d["win"], sink, pos, window=W, ring_cap=ring, out=out, ws=ws_a)

    ms = _graph_time_ms(fn, n_sets)
    nbytes = B * n_cap * (dI + 4) + B * H_I * (dI * 2 + 2) + B * (k + W) * 1024 + B * H * 512 * 2 * 2 + B * k * 4
    gbs = nbytes / (ms * 1e-3) / 1e9
    del sets, out, ws_i, ws_a, topk
    torch.cuda.empty_cache()
    return {"what": "CSA decode (Flash), 32 sequences at 128K context: fp8 indexer 64x128 over 32768 entries, "
                    "top-k 512, attention over 512 entries + 128-token window, 64 heads",
            "ms_per_step": round(ms, 4), "tokens_per_s_per_layer": round(B / (ms * 1e-3), 1),
            "input_sets": n_sets, "roofline": {"bound": "hbm", "bytes": nbytes, "achieved": round(gbs, 1),
                                               "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                               "frac": round(gbs / HBM_PEAK_GBS, 4)}}


def csa_prefill_2k_row(dev):
    """CSA prefill of 2048 tokens (one sequence, 8 heads, indexer 8 x 64 with bf16 keys, top-k 128, sink 0):
    the whole path from raw per-token vectors: block compression with the indexer keys, the window fill,
    the indexer + top-k for all 2048 queries and the attention.  Inputs: N(0,1) hidden states (d = 1024)
    projected by N(0, 0.02^2) weights, drawn on the device.  tokens/s = 2048 / time of the path."""
    import torch
    import long_context_sparse_17_amd as L
    import synth
    T, d, H, H_I, dI, k, W = 2048, 1024, 8, 8, 64, 128, 128
    h = synth.device_normal_f32((T, d), 1.0, 5_000_001)
    proj = lambda n, sd: (h @ synth.device_normal_f32((d, n), 0.02, sd))  # noqa: E731
    kv = proj(512, 5_000_002).to(torch.bfloat16).view(1, T, 512)
    ks = proj(1, 5_000_003).view(1, T).contiguous()
    q = proj(H * 512, 5_000_004).to(torch.bfloat16).view(1, T, H, 512)
    qi = proj(H_I * dI, 5_000_005).to(torch.bfloat16).view(1, T, H_I, dI)
    ik = proj(dI, 5_000_006).to(torch.bfloat16).view(1, T, dI)
    iks = proj(1, 5_000_007).view(1, T).contiguous()
    wi = proj(H_I, 5_000_008).to(torch.bfloat16).view(1, T, H_I)
    sink = torch.zeros(H, dtype=torch.float32, device=dev)
    g = torch.ones(512, dtype=torch.bfloat16, device=dev)
    n_cap = T // 4
    kv_cache = torch.zeros((1, n_cap, 512), dtype=torch.bfloat16, device=dev)
    ik_cache = torch.zeros((1, n_cap, dI), dtype=torch.bfloat16, device=dev)
    win = torch.zeros((1, T, 512), dtype=torch.bfloat16, device=dev)
    pos = torch.arange(T, dtype=torch.int64, device=dev).view(1, T)
    topk = torch.empty((1, T, k), dtype=torch.int32, device=dev)
    out = torch.empty((1, T, H, 512), dtype=torch.bfloat16, device=dev)
    ws_i = L.workspace(L.csa_index_topk_workspace(1, T, n_cap, k), zeroed=True)
    ws_a = L.workspace(L.attend_workspace(1, T, H, k + W))

    def fn(i):
        L.csa_compress_kv(kv, ks, ik, iks, tok0=0, blk_begin=0, n_blk=n_cap, m=4, overlap=4, gamma_kv=g,
                          kv_out=kv_cache, ik_out=ik_cache, ik_fp8=False)
        L.hca_compress_kv(kv, ks, tok0=0, blk_begin=0, n_blk=T, m=1, gamma_kv=g, kv_out=win)
        L.csa_index_topk(qi, wi, ik_cache, None, pos, n_cap=n_cap, m=4, k=k, topk_idx=topk, ws=ws_i)
        L.csa_attend(q, g, kv_cache, topk, win, sink, pos, window=W, ring_cap=0, out=out, ws=ws_a)

    ms = _graph_time_ms(fn, 1, reps=20)
    pairs = sum(t // 4 for t in range(T))
    sel = sum(min(k, t // 4) for t in range(T))
    winkeys = sum(min(W, t + 1) for t in range(T))
    flops = 2.0 * pairs * H_I * dI + 4.0 * 512 * H * (sel + winkeys)
    del h, kv, ks, q, qi, ik, iks, wi, kv_cache, ik_cache, win, topk, out, ws_i, ws_a
    torch.cuda.empty_cache()
    return {"what": "CSA prefill, 2048 tokens, 8 heads, indexer 8x64 bf16, top-k 128 (compress, window, "
                    "indexer + top-k, attention)", "ms_per_call": round(ms, 4),
            "tokens_per_s": round(T / (ms * 1e-3), 1), "flops": flops,
            "achieved_tflops": round(flops / (ms * 1e-3) / 1e12, 2), "bound": "latency (small)"}


def time_stack(layers, steps, warmup, use_graph, ref_y, step=None, outputs=None):
    """Capture one step (default: every layer's step) into a HIP graph (checked bitwise against the
    eager outputs ref_y over three replays; outputs() gives the tensors to compare, default the layers'
    y), then time `steps` replays after `warmup`; eager launches if capture is unavailable.
    Returns (graph or None, ms per step, per-step p10/p50/p90 in ms from a second set of steps)."""
    import torch

    if step is None:
        def step():
            for layer in layers:
                layer.step()
    if outputs is None:
        def outputs():
            return [layer.y for layer in layers]

    graph = None
    if use_graph:
        try:
            s = torch.cuda.Stream()
            s.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(s):
                step()
            torch.cuda.current_stream().wait_stream(s)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                step()
            for _ in range(3):
                for t in outputs():
                    t.zero_()
                g.replay()
                torch.cuda.synchronize()
                if not all(torch.equal(t, r) for t, r in zip(outputs(), ref_y)):
                    raise RuntimeError("graph replay differs from eager")
            graph = g
        except Exception as e:  # graph capture unavailable: time eager launches
            log(f"graph capture not used: {e}")
            graph = None
    run = graph.replay if graph is not None else step
    for _ in range(warmup):
        run()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        run()
    torch.cuda.synchronize()
    ms = (time.perf_counter() - t0) / steps * 1e3
    # per-step spread: events around each of a second set of steps (not part of the timed total)
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    ev[0].record()
    for i in range(steps):
        run()
        ev[i + 1].record()
    torch.cuda.synchronize()
    per = sorted(ev[i].elapsed_time(ev[i + 1]) for i in range(steps))
    spread = {"p10": round(per[len(per) // 10], 4), "p50": round(per[len(per) // 2], 4),
              "p90": round(per[(9 * len(per)) // 10], 4)}
    return graph, ms, spread


def fp8_kv_stack_row(args, dev):
    """The same 4-layer decode step with fp8 K=V storage (cache and ring as E4M3FN codes + row scales):
    tokens/s/layer and the step's algorithmic bytes."""
    import torch
    from long_context_sparse_17_amd.pipeline import hybrid_stack
    layers = hybrid_stack(B=args.batch, ctx=args.ctx, k=1024, device=dev, kv8=True)
    for _ in range(args.warmup):
        for layer in layers:
            layer.step()
    torch.cuda.synchronize()
    ref_y = [layer.y.clone() for layer in layers]
    graph, ms, _ = time_stack(layers, args.steps, args.warmup, not args.no_graph, ref_y)
    nbytes = sum(sum(layer.bytes_per_step().values()) for layer in layers)
    out = {"what": "hybrid 4-layer decode step, fp8 K=V storage", "tokens_per_s_per_layer":
           round(args.batch * len(layers) / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "step_bytes": nbytes, "achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "graph_replay": graph is not None}
    del layers, graph
    torch.cuda.empty_cache()
    return out


def chained_stack_row(args, dev):
    """The 4-layer step as a true stack: input projections of each layer from the hidden state at
    d = 4096 (one pass over the concatenated weights) and the residual h <- h + y after each layer."""
    import torch
    from long_context_sparse_17_amd.pipeline import ChainedStack, hybrid_stack
    layers = hybrid_stack(B=args.batch, ctx=args.ctx, k=1024, device=dev)
    stack = ChainedStack(layers)
    for _ in range(args.warmup):
        stack.step()
    torch.cuda.synchronize()
    ref = [stack.h.clone()]
    graph, ms, _ = time_stack(layers, args.steps, args.warmup, not args.no_graph, ref, step=stack.step,
                           outputs=lambda: [stack.h])
    nbytes = sum(sum(layer.bytes_per_step().values()) for layer in layers) + stack.proj_bytes()
    out = {"what": "hybrid 4-layer decode step chained: input projections from h (d = 4096) + residual",
           "tokens_per_s_per_layer": round(args.batch * len(layers) / (ms * 1e-3), 1), "ms_per_step": round(ms, 4),
           "step_bytes": nbytes, "projection_weight_bytes": sum(w.numel() * 2 for w in stack.w_in),
           "achieved_gbs": round(nbytes / (ms * 1e-3) / 1e9, 1), "graph_replay": graph is not None}
    del stack, layers, graph
    torch.cuda.empty_cache()
    return out


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--batch", type=int, default=8)
    ap.add_argument("--ctx", type=int, default=1 << 20)
    ap.add_argument("--no-graph", action="store_true")
    ap.add_argument("--no-cpu", action="store_true", help="skip the CPU oracle baseline")
    ap.add_argument("--cpu-seqs", type=int, default=2)
    ap.add_argument("--no-fp8kv", action="store_true", help="skip the fp8 K=V variant of the step")
    ap.add_argument("--no-chain", action="store_true", help="skip the chained (projections + residual) variant")
    ap.add_argument("--no-prefill", action="store_true", help="skip the 1M chunked-prefill measurement")
    ap.add_argument("--no-configs", action="store_true", help="skip the HCA 64K, CSA 128K and 2K prefill rows")
    args = ap.parse_args()

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU: the library has no multi-GPU path (the per-GPU kernel is shown at its "
              "real shape; sharding is described in the design notes).", file=sys.stderr)
        sys.exit(2)

    import torch
    import long_context_sparse_17_amd as L
    from long_context_sparse_17_amd.pipeline import CsaDecodeLayer, flops_per_step, hybrid_stack

    L.lib()
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    t_setup = time.perf_counter()
    layers = hybrid_stack(B=args.batch, ctx=args.ctx, k=1024, device=dev)
    torch.cuda.synchronize()
    log(f"setup: caches built in {time.perf_counter() - t_setup:.1f} s")

    def step():
        for layer in layers:
            layer.step()

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    ref_y = [layer.y.clone() for layer in layers]

    graph, ms_per_step, spread = time_stack(layers, args.steps, args.warmup, not args.no_graph, ref_y)
    dt = ms_per_step * 1e-3 * args.steps
    B, nl = args.batch, len(layers)
    value = B * nl / (dt / args.steps)

    # algorithmic bytes of a whole step
    step_bytes = sum(sum(layer.bytes_per_step().values()) for layer in layers)
    step_flops = sum(sum(flops_per_step(layer).values()) for layer in layers)

    # per-kernel durations: a second pass of eager steps with HIP events around every launch
    L.timing_enable(True)
    kt_steps = max(5, min(args.steps, 50))
    for _ in range(kt_steps):
        step()
    torch.cuda.synchronize()
    kernels = {}
    for name in ("index_score_kernel", "topk_filter_kernel", "topk_final_kernel",
                 "attend_csa_kernel", "attend_hca_kernel", "attend_merge_kernel", "out_proj_group_kernel",
                 "out_proj_out_kernel", "compress_kernel", "decode_append_kernel", "input_proj_kernel"):
        ms, n = L.timing_read(name)
        if n:
            kernels[name] = {"avg_us": round(ms / n * 1e3, 3), "launches_per_step": n // kt_steps}
    L.timing_enable(False)
    # attention against the HBM roofline, per layer type (bytes of one launch: the layer's keys, q, o)
    attention = {}
    for layer in layers[:2]:
        kind = "csa" if isinstance(layer, CsaDecodeLayer) else "hca"
        name = f"attend_{kind}_kernel"
        if name in kernels:
            nb = layer.bytes_per_step()["attend"]
            us = kernels[name]["avg_us"]
            gb = nb / (us * 1e-6) / 1e9
            attention[kind] = {"kernel": name, "bytes_per_launch": nb, "avg_us": us, "achieved": round(gb, 1),
                               "unit": "GB/s", "frac": round(gb / HBM_PEAK_GBS, 4)}
            if "attend_merge_kernel" in kernels:
                usm = us + kernels["attend_merge_kernel"]["avg_us"]
                attention[kind]["with_merge_us"] = round(usm, 3)
                attention[kind]["with_merge_frac"] = round(nb / (usm * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)

    csa = [layer for layer in layers if isinstance(layer, CsaDecodeLayer)]
    idx_bytes = csa[0].bytes_per_step()["index"]             # per launch: every visible fp8 key + scale once
    idx_us = kernels["index_score_kernel"]["avg_us"]
    achieved = idx_bytes / (idx_us * 1e-6) / 1e9
    roofline = {"bound": "hbm", "kernel": "index_score_kernel", "achieved": round(achieved, 1),
                "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                "traffic": stored_traffic(), "bytes_per_launch": idx_bytes, "avg_us": idx_us}
    per_kernel_gbs = {}
    if "out_proj_out_kernel" in kernels:
        wb = layers[0].w_o.numel() * 2
        per_kernel_gbs["out_proj_out_kernel"] = round(wb / (kernels["out_proj_out_kernel"]["avg_us"] * 1e-6) / 1e9, 1)
        wb = layers[0].w_g.numel() * 2
        per_kernel_gbs["out_proj_group_kernel"] = round(wb / (kernels["out_proj_group_kernel"]["avg_us"] * 1e-6) / 1e9, 1)

    # reference: a plain device-to-device copy of 1 GiB (read + write bytes / time)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev)
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(10):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbs = 2 * (1 << 30) * 10 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    mfma_tflops = mfma_reference(dev)
    next_rows = {"decode_append": decode_append_rows(dev, B), "mhc_mix": mhc_row(dev)}
    if not args.no_fp8kv:
        next_rows["fp8_kv"] = fp8_kv_stack_row(args, dev)
    if not args.no_chain:
        next_rows["chained_stack"] = chained_stack_row(args, dev)
    prefill = None if args.no_prefill else prefill_row(dev)
    configs = None
    if not args.no_configs:
        configs = {"hca_decode_64k": hca_decode_64k_row(dev), "csa_decode_128k": csa_decode_128k_row(dev),
                   "csa_prefill_2k": csa_prefill_2k_row(dev)}
    roofline["frac_of_copy"] = round(achieved / copy_gbs, 4)

    cpu = None
    fp8_check = None
    if not args.no_cpu:
        rate, secs, threads, sample, single = cpu_baseline(layers, args.cpu_seqs)
        cpu = {"value": round(rate, 3), "unit": "tokens/s/layer", "cores": threads, "kind": "oracle",
               "sample": sample, "seconds": round(secs, 2), "single_thread": single}
        fp8_check = fp8_indexer_check(dev)

    out = {
        "metric": METRIC, "value": round(value, 1), "unit": "tokens/s/layer", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_per_step, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": "hybrid4_decode_1m", "layers": ["csa", "hca", "csa", "hca"], "batch": B,
                   "ctx": args.ctx, "heads": 64, "head_dim": 512, "window": 128, "topk": 1024,
                   "indexer": "64x128 fp8_e4m3", "m_csa": 4, "m_hca": 128, "g": 8, "d_g": 1024, "d": 4096,
                   "graph_replay": graph is not None},
        "roofline": roofline,
        "step_ms_spread": spread,
        "step_hbm": {"bytes": step_bytes, "achieved_gbs": round(step_bytes / (ms_per_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                     "flops": step_flops},
        "kernels_event_timed": kernels,
        "kernels_note": "eager launches, each bracketed by HIP events on its stream (the events add about 2 us "
                        "per launch): per-kernel durations, not a breakdown of the graph-replayed step",
        "attention_roofline": attention, "kernel_gbs": per_kernel_gbs, "hbm_copy_gbs": round(copy_gbs, 1),
        "mfma_gemm_bf16_tflops": round(mfma_tflops, 1), "next": next_rows, "prefill_1m": prefill,
        "configs": configs, "fp8_indexer_vs_exact": fp8_check, "cpu_baseline": cpu,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
