"""GPU parity of kv_decode_append, the per-token decode path of the compressed-KV state, in a
continuous-batching loop: sequences start at different steps, pause (position -1) and stop, so the
batch is ragged at every step.  After the loop every finished block's entry (and indexer key) must
equal the oracle's compression of that sequence's token stream, the window ring must hold the last
tokens normed and rotated, and untouched rows must stay untouched.  The state buffer starts as NaN
bytes: the first token of a block starts its state, so nothing is read before it is written.
"""
import numpy as np
import pytest
import torch

import long_context_sparse_17_amd as L
import oracle as O
import synth
from lcs_testutil import assert_close, errors, from_bits, to_np_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"
RING = 160


def _schedule(B, steps, m):
    """Per step and sequence: the token index appended, or -1.  Sequence 0 runs throughout, 1 starts
    late, 2 pauses for a while, 3 stops early, 4 starts late and pauses."""
    pos = np.full((steps, B), -1, dtype=np.int64)
    start = [0, 9, 0, 0, 37]
    stop = [steps, steps, steps, 100, steps]
    pause = {2: range(100, 131), 4: range(150, 170)}
    for b in range(B):
        n = 0
        for s in range(start[b], stop[b]):
            if b in pause and s in pause[b]:
                continue
            pos[s, b] = n
            n += 1
    return pos


@pytest.mark.parametrize("mode", ["csa_fp8", "csa_bf16", "hca", "csa_ov2"])
def test_decode_append_serving_loop(mode):
    m, ov, dI, fp8 = {"csa_fp8": (4, 4, 128, True), "csa_bf16": (4, 4, 64, False), "hca": (128, 0, 0, False),
                      "csa_ov2": (4, 2, 128, True)}[mode]
    B, steps, off = 5, 300, 4321
    cfg = 60 + len(mode)
    kv = synth.normal_bf16((B, steps, 512), 1.28, cfg, 1)
    ks = synth.normal_f32((B, steps), 1.28, cfg, 2)
    ik = synth.normal_bf16((B, steps, max(dI, 64)), 1.28, cfg, 3)
    iks = synth.normal_f32((B, steps), 1.28, cfg, 4)
    gamma = synth.f32_to_bf16_bits(0.5 + synth.rng(cfg, 5).random(512, dtype=np.float32))
    pos = _schedule(B, steps, m)
    n_tok = (pos.max(axis=0) + 1).astype(int)

    # per-step inputs: the token each sequence appends (zeros where inactive)
    idx = np.where(pos >= 0, pos, 0)
    b_ix = np.arange(B)[None, :]
    step_kv = from_bits(np.ascontiguousarray(kv[b_ix, idx]))                     # [steps, B, 512]
    step_ks = torch.from_numpy(np.ascontiguousarray(ks[b_ix, idx])).to(DEV)
    step_ik = from_bits(np.ascontiguousarray(ik[b_ix, idx])) if dI else None
    step_iks = torch.from_numpy(np.ascontiguousarray(iks[b_ix, idx])).to(DEV) if dI else None
    step_pos = torch.from_numpy(pos).to(DEV)

    nb_cap = steps // m + 2
    state = torch.full((L.kv_decode_state_bytes(B) // 4,), float("nan"), dtype=torch.float32, device=DEV)
    ring = torch.zeros((B, RING, 512), dtype=torch.bfloat16, device=DEV)
    kv_out = torch.zeros((B, nb_cap, 512), dtype=torch.bfloat16, device=DEV)
    ik_out = ik_sc = None
    if dI:
        ik_out = torch.zeros((B, nb_cap, dI), dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
        ik_sc = torch.zeros((B, nb_cap), dtype=torch.float32, device=DEV)
    g_dev = from_bits(gamma)
    for s in range(steps):
        L.kv_decode_append(step_kv[s], step_ks[s], step_ik[s] if dI else None, step_iks[s] if dI else None,
                           step_pos[s], m=m, overlap=ov, gamma_kv=g_dev, state=state, kv_out=kv_out, win=ring,
                           ring_cap=RING, ik_out=ik_out, ik_scale=ik_sc, ik_fp8=fp8, rope_offset=off)
    torch.cuda.synchronize()

    g64 = synth.bf16_bits_to_f64(gamma)
    got_kv = to_np_bf16(kv_out)
    got_ring = to_np_bf16(ring)
    for b in range(B):
        n = int(n_tok[b])
        nb = n // m
        x = synth.bf16_bits_to_f64(kv[b, :n])
        ref = O.compress_kv(x, ks[b, :n].astype(np.float64), m, ov, g64, 1e-6, 10000.0, off)[:nb]
        assert_close(got_kv[b, :nb], ref, f"{mode} entries b={b}")
        assert np.all(got_kv[b, nb:] == 0), "rows of unfinished blocks must not be written"
        win = O.window_entries(x, g64, 1e-6, 10000.0, off)
        last = range(max(0, n - RING), n)
        assert_close(got_ring[b, [j % RING for j in last]], win[list(last)], f"{mode} ring b={b}")
        if dI:
            e = O.pool(synth.bf16_bits_to_f64(ik[b, :n, :dI]), iks[b, :n].astype(np.float64), m, ov)[:nb]
            if fp8:
                codes, sc, deq = O.fp8_quantize_rows(e)
                np.testing.assert_allclose(ik_sc[b, :nb].cpu().numpy(), sc, rtol=1e-5)
                gc = ik_out[b, :nb].cpu().numpy().astype(int)
                diff = np.abs((gc & 0x7F) - (codes.astype(int) & 0x7F))
                assert diff.max() <= 1                       # fp32 online vs fp64 pooling: one code apart at most
                assert (diff > 0).mean() < 0.01
                got = O.e4m3_decode(ik_out[b, :nb].cpu().numpy()) * ik_sc[b, :nb].cpu().numpy()[:, None]
                assert errors(got, deq)[1] < 1e-2
            else:
                assert_close(to_np_bf16(ik_out[b, :nb]), e, f"{mode} bf16 keys b={b}")

    # the bulk path on the same streams agrees with the per-token path
    b = 0
    n = int(n_tok[b])
    nb = n // m
    bulk = torch.zeros((1, nb_cap, 512), dtype=torch.bfloat16, device=DEV)
    if dI:
        L.csa_compress_kv(from_bits(kv[b:b + 1, :n]), torch.from_numpy(ks[b:b + 1, :n].copy()).to(DEV),
                          from_bits(np.ascontiguousarray(ik[b:b + 1, :n, :dI])),
                          torch.from_numpy(iks[b:b + 1, :n].copy()).to(DEV), tok0=0, blk_begin=0, n_blk=nb, m=m,
                          overlap=ov, gamma_kv=g_dev, kv_out=bulk,
                          ik_out=torch.zeros((1, nb_cap, dI), dtype=ik_out.dtype, device=DEV),
                          ik_scale=torch.zeros((1, nb_cap), dtype=torch.float32, device=DEV), ik_fp8=fp8,
                          rope_offset=off)
    else:
        L.hca_compress_kv(from_bits(kv[b:b + 1, :n]), torch.from_numpy(ks[b:b + 1, :n].copy()).to(DEV), tok0=0,
                          blk_begin=0, n_blk=nb, m=m, gamma_kv=g_dev, kv_out=bulk, rope_offset=off)
    torch.cuda.synchronize()
    assert_close(got_kv[b, :nb], to_np_bf16(bulk[0, :nb]), f"{mode} per-token vs bulk")


def _fp8_rows_match(codes, scales, ref, what):
    """fp8 rows written from fp32 values against the oracle's quantisation of its fp64 values:
    scales to fp32 rounding, codes at most one step apart (< 1 % of them), dequantised rel-L2 < 1e-2."""
    rc, rs, rdeq = O.fp8_quantize_rows(ref)
    np.testing.assert_allclose(scales, rs, rtol=1e-5, err_msg=what)
    diff = np.abs((codes.astype(int) & 0x7F) - (rc.astype(int) & 0x7F))
    assert diff.max() <= 1 and (diff > 0).mean() < 0.01, what
    got = O.e4m3_decode(codes) * scales[:, None].astype(np.float64)
    assert errors(got, rdeq)[1] < 1e-2, what


@pytest.mark.parametrize("m,ov", [(4, 4), (128, 0)])
def test_decode_append_fp8_kv_rows(m, ov):
    """The same serving loop with fp8 K=V storage: entries and ring rows as E4M3FN codes + scales."""
    B, steps, off = 5, 300, 99
    cfg = 170 + m
    kv = synth.normal_bf16((B, steps, 512), 1.28, cfg, 1)
    ks = synth.normal_f32((B, steps), 1.28, cfg, 2)
    gamma = synth.f32_to_bf16_bits(0.5 + synth.rng(cfg, 5).random(512, dtype=np.float32))
    pos = _schedule(B, steps, m)
    n_tok = (pos.max(axis=0) + 1).astype(int)
    idx = np.where(pos >= 0, pos, 0)
    b_ix = np.arange(B)[None, :]
    step_kv = from_bits(np.ascontiguousarray(kv[b_ix, idx]))
    step_ks = torch.from_numpy(np.ascontiguousarray(ks[b_ix, idx])).to(DEV)
    step_pos = torch.from_numpy(pos).to(DEV)
    nb_cap = steps // m + 2
    state = torch.zeros(L.kv_decode_state_bytes(B), dtype=torch.uint8, device=DEV)
    ring = torch.zeros((B, RING, 512), dtype=torch.uint8, device=DEV)
    ring_sc = torch.zeros((B, RING), dtype=torch.float32, device=DEV)
    kv_out = torch.zeros((B, nb_cap, 512), dtype=torch.uint8, device=DEV)
    kv_sc = torch.zeros((B, nb_cap), dtype=torch.float32, device=DEV)
    g_dev = from_bits(gamma)
    for s in range(steps):
        L.kv_decode_append(step_kv[s], step_ks[s], None, None, step_pos[s], m=m, overlap=ov, gamma_kv=g_dev,
                           state=state, kv_out=kv_out, kv_scale=kv_sc, win=ring, win_scale=ring_sc, ring_cap=RING,
                           rope_offset=off)
    torch.cuda.synchronize()
    g64 = synth.bf16_bits_to_f64(gamma)
    codes, sc = kv_out.cpu().numpy(), kv_sc.cpu().numpy()
    rcodes, rsc = ring.cpu().numpy(), ring_sc.cpu().numpy()
    for b in range(B):
        n = int(n_tok[b])
        nb = n // m
        x = synth.bf16_bits_to_f64(kv[b, :n])
        if nb:
            ref = O.compress_kv(x, ks[b, :n].astype(np.float64), m, ov, g64, 1e-6, 10000.0, off)[:nb]
            _fp8_rows_match(codes[b, :nb], sc[b, :nb], ref, f"fp8 entries b={b}")
        assert np.all(codes[b, nb:] == 0) and np.all(sc[b, nb:] == 0)
        win = O.window_entries(x, g64, 1e-6, 10000.0, off)
        last = list(range(max(0, n - RING), n))
        rows = [j % RING for j in last]
        _fp8_rows_match(rcodes[b, rows], rsc[b, rows], win[last], f"fp8 ring b={b}")


@pytest.mark.parametrize("m,ov", [(4, 4), (128, 0), (4, 2)])
def test_decode_append_resumes_mid_stream(m, ov):
    """Sequences resumed at t0 > 0 on zero-filled slots: blocks whose first token comes before t0 are
    left alone (their rows stay as they were); every block that starts at or after t0 and ends
    within the appended tokens is written and equals the oracle's."""
    B, n, off = 2, 300, 77
    t0s = np.array([1001, 37], dtype=np.int64)
    cfg = 80 + m + ov
    T = int(t0s.max()) + n
    kv = synth.normal_bf16((B, T, 512), 1.28, cfg, 1)
    ks = synth.normal_f32((B, T), 1.28, cfg, 2)
    gamma = synth.f32_to_bf16_bits(0.5 + synth.rng(cfg, 5).random(512, dtype=np.float32))
    nb_cap = T // m + 2
    state = torch.zeros(L.kv_decode_state_bytes(B), dtype=torch.uint8, device=DEV)
    ring = torch.zeros((B, RING, 512), dtype=torch.bfloat16, device=DEV)
    kv_out = torch.zeros((B, nb_cap, 512), dtype=torch.bfloat16, device=DEV)
    g_dev = from_bits(gamma)
    for j in range(n):
        p = t0s + j
        L.kv_decode_append(from_bits(np.ascontiguousarray(kv[np.arange(B), p])),
                           torch.from_numpy(np.ascontiguousarray(ks[np.arange(B), p])).to(DEV),
                           None, None, torch.from_numpy(p).to(DEV), m=m, overlap=ov, gamma_kv=g_dev, state=state,
                           kv_out=kv_out, win=ring, ring_cap=RING, rope_offset=off)
    torch.cuda.synchronize()
    g64 = synth.bf16_bits_to_f64(gamma)
    got = to_np_bf16(kv_out)
    for b in range(B):
        t0, t1 = int(t0s[b]), int(t0s[b]) + n            # appended positions [t0, t1)
        first = lambda j: max(0, j * m - ov)              # noqa: E731
        done = [j for j in range(nb_cap) if first(j) >= t0 and (j + 1) * m <= t1]
        assert done, "the test must finish blocks"
        x = synth.bf16_bits_to_f64(kv[b, :t1])
        x[:t0] = 0.0                                      # tokens never appended take no part
        ref = O.compress_kv(x, ks[b, :t1].astype(np.float64), m, ov, g64, 1e-6, 10000.0, off)
        assert_close(got[b, done], ref[done], f"resumed entries b={b} m={m} ov={ov}")
        untouched = [j for j in range(nb_cap) if j not in done]
        assert np.all(got[b, untouched] == 0), "blocks opened before the first append must not be written"


def test_decode_append_inactive_batch_touches_nothing():
    B = 3
    kv = synth.normal_bf16((B, 512), 1.28, 71, 1)
    state = torch.full((L.kv_decode_state_bytes(B) // 4,), 7.0, dtype=torch.float32, device=DEV)
    ring = torch.full((B, 8, 512), 3.0, dtype=torch.bfloat16, device=DEV)
    out = torch.full((B, 4, 512), 5.0, dtype=torch.bfloat16, device=DEV)
    pos = torch.full((B,), -1, dtype=torch.int64, device=DEV)
    L.kv_decode_append(from_bits(kv), torch.zeros(B, device=DEV), None, None, pos, m=1, overlap=0,
                       gamma_kv=from_bits(synth.f32_to_bf16_bits(np.ones(512, np.float32))), state=state,
                       kv_out=out, win=ring, ring_cap=8)
    torch.cuda.synchronize()
    assert torch.all(state == 7.0) and torch.all(ring == 3.0) and torch.all(out == 5.0)


@pytest.mark.parametrize("kv8", [False, True])
def test_index_topk_append_matches_separate_calls(kv8):
    """csa_index_topk_append (the append run beside the decode selection's final kernel) leaves every
    buffer bit for bit as kv_decode_append followed by csa_index_topk: selections, pooling state, ring
    rows, finished entries and indexer keys.  Sequences at a block-ending token, mid-block, at a block
    start, inactive (position -1), with the open blocks primed by earlier appends."""
    B, m, ov, dI, H_I, k, n_cap, ring = 6, 4, 4, 128, 64, 64, 600, 256
    t_step = np.array([2399, 2397, -1, 1203, 2000, 1204], dtype=np.int64)
    cfg = 71
    gamma = from_bits(synth.normal_bf16((512,), 1.0, cfg, 1))
    kv8_dt = torch.uint8 if kv8 else torch.bfloat16
    kv_out = torch.zeros((B, n_cap, 512), dtype=kv8_dt, device=DEV)
    win = torch.zeros((B, ring, 512), dtype=kv8_dt, device=DEV)
    kv_sc = torch.zeros((B, n_cap), dtype=torch.float32, device=DEV) if kv8 else None
    win_sc = torch.zeros((B, ring), dtype=torch.float32, device=DEV) if kv8 else None
    ik = torch.from_numpy(synth.fp8_codes((B, n_cap, dI), cfg, 2)).to(DEV)
    iks = torch.from_numpy(synth.positive_scales((B, n_cap), cfg, 3)).to(DEV)
    state = torch.zeros(L.kv_decode_state_bytes(B), dtype=torch.uint8, device=DEV)
    akw = dict(m=m, overlap=ov, gamma_kv=gamma, state=state, kv_out=kv_out, win=win, ring_cap=ring, ik_out=ik,
               ik_scale=iks, ik_fp8=True, kv_scale=kv_sc, win_scale=win_sc)

    def tokens(seed):
        return (from_bits(synth.normal_bf16((B, 512), 1.28, cfg, seed)), torch.from_numpy(
                synth.normal_f32((B,), 1.28, cfg, seed + 1)).to(DEV),
                from_bits(synth.normal_bf16((B, dI), 1.28, cfg, seed + 2)), torch.from_numpy(
                synth.normal_f32((B,), 1.28, cfg, seed + 3)).to(DEV))

    # prime the open blocks: the 7 tokens before each position, one append per token
    for j in range(7, 0, -1):
        pos = torch.from_numpy(np.where(t_step >= j, t_step - j, -1)).to(DEV)
        L.kv_decode_append(*tokens(10 + 4 * j), pos, **akw)
    pos = torch.from_numpy(t_step).to(DEV)
    q_pos = pos.view(B, 1).clone()
    q_idx = from_bits(synth.normal_bf16((B, 1, H_I, dI), 1.28, cfg, 60))
    w_idx = from_bits(synth.normal_bf16((B, 1, H_I), 1.28, cfg, 61))
    tok = tokens(70)
    ws = L.workspace(L.csa_index_topk_workspace(B, 1, n_cap, k), zeroed=True)
    bufs = [state, kv_out, win, ik, iks] + ([kv_sc, win_sc] if kv8 else [])
    start = [t.clone() for t in bufs]

    sel_a = torch.full((B, 1, k), -7, dtype=torch.int32, device=DEV)
    L.kv_decode_append(*tok, pos, **akw)
    L.csa_index_topk(q_idx, w_idx, ik, iks, q_pos, n_cap=n_cap, m=m, k=k, topk_idx=sel_a, ws=ws)
    torch.cuda.synchronize()
    after_a = [t.clone() for t in bufs]

    for t, s0 in zip(bufs, start):
        t.copy_(s0)
    sel_b = torch.full((B, 1, k), -7, dtype=torch.int32, device=DEV)
    L.csa_index_topk_append(q_idx, w_idx, ik, iks, q_pos, n_cap=n_cap, m=m, k=k, topk_idx=sel_b, ws=ws,
                            append=dict(kv_tok=tok[0], kv_score=tok[1], ik_tok=tok[2], ik_score=tok[3], pos=pos, **akw))
    torch.cuda.synchronize()
    assert torch.equal(sel_a, sel_b)
    for name, a, b in zip(["state", "kv_out", "win", "ik", "iks", "kv_sc", "win_sc"], after_a, bufs):
        assert torch.equal(a, b), f"{name} differs between the fused and the separate calls"
    # the step wrote what it should: the ring rows of the active sequences, and the entries of the
    # blocks that end at their token (t = 2399 -> entry 599, t = 1203 -> entry 300)
    for b in range(B):
        t = int(t_step[b])
        changed = not torch.equal(win[b, t % ring], start[2][b, t % ring]) if t >= 0 else False
        assert changed == (t >= 0), f"ring row of sequence {b}"
    assert not torch.equal(kv_out[0, 599], start[1][0, 599]) and not torch.equal(kv_out[3, 300], start[1][3, 300])
    assert torch.equal(kv_out[1], start[1][1]) and torch.equal(kv_out[4], start[1][4])
    assert int(ws[:L.lib().csa_index_topk_state_bytes()].count_nonzero()) == 0   # zero state kept


@pytest.mark.parametrize("kv8", [False, True])
def test_hca_attend_append_matches_separate_calls(kv8):
    """hca_attend_append (the append's workgroups in the attention's launch, the query's own window
    row formed by the split that holds it) gives bit for bit kv_decode_append followed by hca_attend:
    outputs, pooling state, ring rows and entries.  Sequences at a block-ending token, mid-block and
    inactive (position -1: the query then reads its window row as stored), many splits."""
    B, m, H, n_cap, ring, W = 5, 128, 64, 64, 256, 128
    t_step = np.array([64 * 128 - 1, 5000, -1, 2 * 128 - 1, 7000], dtype=np.int64)
    cfg = 72
    gamma = from_bits(synth.normal_bf16((512,), 1.0, cfg, 1))
    kv8_dt = torch.uint8 if kv8 else torch.bfloat16
    kv_out = torch.zeros((B, n_cap, 512), dtype=kv8_dt, device=DEV)
    win = torch.zeros((B, ring, 512), dtype=kv8_dt, device=DEV)
    kv_sc = torch.ones((B, n_cap), dtype=torch.float32, device=DEV) if kv8 else None
    win_sc = torch.ones((B, ring), dtype=torch.float32, device=DEV) if kv8 else None
    state = torch.zeros(L.kv_decode_state_bytes(B), dtype=torch.uint8, device=DEV)
    akw = dict(m=m, overlap=0, gamma_kv=gamma, state=state, kv_out=kv_out, win=win, ring_cap=ring, kv_scale=kv_sc,
               win_scale=win_sc)

    def tokens(seed):
        return (from_bits(synth.normal_bf16((B, 512), 1.28, cfg, seed)),
                torch.from_numpy(synth.normal_f32((B,), 1.28, cfg, seed + 1)).to(DEV))

    # fill the caches and rings with earlier tokens: the last 150 tokens before each position one by
    # one (the window and the open block), the older entries drawn directly
    if kv8:
        kv_out.copy_(torch.from_numpy(synth.fp8_codes((B, n_cap, 512), cfg, 3)))
        kv_sc.copy_(torch.from_numpy(synth.positive_scales((B, n_cap), cfg, 4)))
    else:
        kv_out.copy_(from_bits(synth.normal_bf16((B, n_cap, 512), 1.0, cfg, 3)))
    for j in range(150, 0, -1):
        pos = torch.from_numpy(np.where(t_step >= j, t_step - j, -1)).to(DEV)
        kt, ks = tokens(100 + 2 * j)
        L.kv_decode_append(kt, ks, None, None, pos, **akw)
    pos = torch.from_numpy(t_step).to(DEV)
    q_pos = pos.view(B, 1).clone()
    q = from_bits(synth.normal_bf16((B, 1, H, 512), 1.28, cfg, 60))
    sink = torch.from_numpy(synth.normal_f32((H,), 1.0, cfg, 61)).to(DEV)
    kt, ks = tokens(70)
    ws = L.workspace(L.attend_workspace(B, 1, H, n_cap + W))
    bufs = [state, kv_out, win] + ([kv_sc, win_sc] if kv8 else [])
    start = [t.clone() for t in bufs]
    extra = dict(kv_scale=kv_sc, win_scale=win_sc) if kv8 else {}

    out_a = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
    L.kv_decode_append(kt, ks, None, None, pos, **akw)
    L.hca_attend(q, gamma, kv_out, win, sink, q_pos, n_cap=n_cap, m=m, window=W, ring_cap=ring, out=out_a, ws=ws,
                 **extra)
    torch.cuda.synchronize()
    after_a = [t.clone() for t in bufs]

    for t, s0 in zip(bufs, start):
        t.copy_(s0)
    out_b = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
    L.hca_attend_append(q, gamma, sink, q_pos, n_cap=n_cap, window=W, out=out_b, ws=ws,
                        append=dict(kv_tok=kt, kv_score=ks, ik_tok=None, ik_score=None, pos=pos, **akw))
    torch.cuda.synchronize()
    active = t_step >= 0
    assert torch.equal(out_a[torch.from_numpy(active)], out_b[torch.from_numpy(active)])
    for name, a, b in zip(["state", "kv_out", "win", "kv_sc", "win_sc"], after_a, bufs):
        assert torch.equal(a, b), f"{name} differs between the fused and the separate calls"
    # the query's own row is the last window key: the ring row the append wrote is the one scored
    for b in range(B):
        t = int(t_step[b])
        if t >= 0:
            assert not torch.equal(win[b, t % ring], start[2][b, t % ring])
    assert not torch.equal(kv_out[0, 63], start[1][0, 63]) and not torch.equal(kv_out[3, 1], start[1][3, 1])
