"""GPU parity of every C-ABI entry point against the fp64 oracle on small seeded inputs.

Sizes span several tiles / chunks and a ragged tail; edge cases: n_vis = 0, n_vis < k, ties,
-1 padding, ring-buffer windows, one split and many splits, heads < 16.
"""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_17_amd as L
import oracle as O
import synth
from lcs_testutil import (assert_close, check_topk_row, errors, from_bits,
                          index_oracle_row, to_np_bf16)

pytestmark = pytest.mark.gpu
DEV = "cuda"


def dev_f32(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def dev_i64(a):
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.int64)).to(DEV)


# ----------------------------------------------------------------------------------- fp8 quantiser
def test_fp8_quantiser_bit_exact_exhaustive():
    """Every bf16 value in [-448, 448] through the device quantiser (m = 1 compression of the
    indexer key, scale exactly 1) against the oracle's E4M3FN encoder; plus random rows."""
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = synth.bf16_bits_to_f32(bits)
    keep = np.isfinite(v) & (np.abs(v) <= 448.0)
    bits = bits[keep]
    per = 127
    R = (bits.size + per - 1) // per
    pad = np.full(R * per - bits.size, bits[0], dtype=np.uint16)
    rows = np.concatenate([bits, pad]).reshape(R, per)
    rows = np.concatenate([rows, np.full((R, 1), synth.f32_to_bf16_bits(np.float32(448.0)), np.uint16)], 1)
    rnd = synth.normal_bf16((64, 128), 1.28, 900, 1)
    ik_bits = np.concatenate([rows, rnd], 0)
    T = ik_bits.shape[0]
    ik = from_bits(ik_bits[None])
    kv = torch.zeros((1, T, 512), dtype=torch.bfloat16, device=DEV)
    zs = torch.zeros((1, T), dtype=torch.float32, device=DEV)
    gamma = torch.ones(512, dtype=torch.bfloat16, device=DEV)
    kv_out = torch.empty((1, T, 512), dtype=torch.bfloat16, device=DEV)
    ik_out = torch.empty((1, T, 128), dtype=torch.uint8, device=DEV)
    ik_sc = torch.empty((1, T), dtype=torch.float32, device=DEV)
    L.csa_compress_kv(kv, zs, ik, zs, tok0=0, blk_begin=0, n_blk=T, m=1, overlap=0, gamma_kv=gamma,
                      kv_out=kv_out, ik_out=ik_out, ik_scale=ik_sc, ik_fp8=True)
    torch.cuda.synchronize()
    codes, s, _ = O.fp8_quantize_rows(synth.bf16_bits_to_f64(ik_bits), kernel_fp32=True)
    got = ik_out[0].cpu().numpy()
    np.testing.assert_array_equal(ik_sc[0].cpu().numpy(), s.astype(np.float32))
    np.testing.assert_array_equal(got, codes)


# ----------------------------------------------------------------------------------- compression
def _compress_inputs(B, T, dI, cfg):
    kv = synth.normal_bf16((B, T, 512), 1.28, cfg, 1)
    ks = synth.normal_f32((B, T), 1.28, cfg, 2)
    ik = synth.normal_bf16((B, T, dI), 1.28, cfg, 3)
    iks = synth.normal_f32((B, T), 1.28, cfg, 4)
    gamma = synth.f32_to_bf16_bits(0.5 + synth.rng(cfg, 5).random(512, dtype=np.float32))
    return kv, ks, ik, iks, gamma


@pytest.mark.parametrize("fp8", [True, False])
def test_csa_compress_parity(fp8):
    B, T, m, ov, dI = 2, 777, 4, 4, 128 if fp8 else 64
    kv, ks, ik, iks, gamma = _compress_inputs(B, T, dI, 11)
    nb = T // m
    kv_out = torch.zeros((B, nb + 3, 512), dtype=torch.bfloat16, device=DEV)
    ik_out = torch.zeros((B, nb + 3, dI), dtype=torch.uint8 if fp8 else torch.bfloat16, device=DEV)
    ik_sc = torch.zeros((B, nb + 3), dtype=torch.float32, device=DEV)
    off = 4321
    # first half from all columns, second half from a column window that starts later (tok0 > 0)
    h = nb // 2
    L.csa_compress_kv(from_bits(kv), dev_f32(ks), from_bits(ik), dev_f32(iks), tok0=0, blk_begin=0, n_blk=h, m=m,
                      overlap=ov, gamma_kv=from_bits(gamma), kv_out=kv_out, ik_out=ik_out,
                      ik_scale=ik_sc if fp8 else None, ik_fp8=fp8, rope_offset=off)
    t0 = h * m - ov
    L.csa_compress_kv(from_bits(kv[:, t0:]), dev_f32(ks[:, t0:]), from_bits(ik[:, t0:]), dev_f32(iks[:, t0:]),
                      tok0=t0, blk_begin=h, n_blk=nb - h, m=m, overlap=ov, gamma_kv=from_bits(gamma),
                      kv_out=kv_out, ik_out=ik_out, ik_scale=ik_sc if fp8 else None, ik_fp8=fp8,
                      rope_offset=off)
    torch.cuda.synchronize()
    g64 = synth.bf16_bits_to_f64(gamma)
    for b in range(B):
        x = synth.bf16_bits_to_f64(kv[b])
        ref = O.compress_kv(x, ks[b].astype(np.float64), m, ov, g64, 1e-6, 10000.0, off)
        assert_close(to_np_bf16(kv_out[b, :nb]), ref, f"kv entries b={b}")
        e = O.pool(synth.bf16_bits_to_f64(ik[b]), iks[b].astype(np.float64), m, ov)
        if fp8:
            codes, s, deq = O.fp8_quantize_rows(e)
            got = O.e4m3_decode(ik_out[b, :nb].cpu().numpy()) * ik_sc[b, :nb].cpu().numpy()[:, None]
            np.testing.assert_allclose(ik_sc[b, :nb].cpu().numpy(), s, rtol=1e-5)
            gc = ik_out[b, :nb].cpu().numpy().astype(int)
            diff = np.abs((gc & 0x7F) - (codes.astype(int) & 0x7F))
            assert diff.max() <= 1                          # fp32 vs fp64 pooling: at most one code apart
            assert (diff > 0).mean() < 0.01
            _, rl = errors(got, deq)
            assert rl < 1e-2
        else:
            assert_close(to_np_bf16(ik_out[b, :nb]), e, f"bf16 indexer keys b={b}")


def test_hca_compress_and_window_ring_parity():
    B, T = 3, 600
    kv, ks, _, _, gamma = _compress_inputs(B, T, 64, 12)
    g64 = synth.bf16_bits_to_f64(gamma)
    nb = T // 128
    out = torch.zeros((B, nb, 512), dtype=torch.bfloat16, device=DEV)
    L.hca_compress_kv(from_bits(kv), dev_f32(ks), tok0=0, blk_begin=0, n_blk=nb, m=128, gamma_kv=from_bits(gamma),
                      kv_out=out)
    # window fill into a ring of 160 rows: tokens 280..599 in two calls of 160 (the second overwrites)
    ring = torch.zeros((B, 160, 512), dtype=torch.bfloat16, device=DEV)
    for t0 in (280, 440):
        L.hca_compress_kv(from_bits(kv[:, t0:]), dev_f32(ks[:, t0:]), tok0=t0, blk_begin=t0, n_blk=160, m=1,
                          gamma_kv=from_bits(gamma), kv_out=ring, ring_cap=160)
    with pytest.raises(L.LcsError):
        L.hca_compress_kv(from_bits(kv[:, 200:]), dev_f32(ks[:, 200:]), tok0=200, blk_begin=200, n_blk=161, m=1,
                          gamma_kv=from_bits(gamma), kv_out=ring, ring_cap=160)
    torch.cuda.synchronize()
    for b in range(B):
        x = synth.bf16_bits_to_f64(kv[b])
        assert_close(to_np_bf16(out[b]), O.compress_kv(x, ks[b], 128, 0, g64), f"hca entries b={b}")
        win = O.window_entries(x, g64)
        got = to_np_bf16(ring[b])
        ref = np.stack([win[j] for j in range(440, 600)])
        rows = np.array([j % 160 for j in range(440, 600)])
        assert_close(got[rows], ref, f"window ring b={b}")


# ----------------------------------------------------------------------------------- indexer + top-k
def _index_case(B, Tq, n_cap, H_I, dI, k, m, fp8, positions, cfg, ties=False, mutate=None, return_idx=False):
    q = synth.normal_bf16((B, Tq, H_I, dI), 1.28, cfg, 21)
    w = synth.normal_bf16((B, Tq, H_I), 1.28, cfg, 22)
    ik_ld = n_cap + 5
    if fp8:
        codes = synth.fp8_codes((B, ik_ld, dI), cfg, 23)
        scale = synth.positive_scales((B, ik_ld), cfg, 24)
        if ties:
            codes[:, : n_cap // 2] = codes[:, :1]
            scale[:, : n_cap // 2] = scale[:, :1]
        if mutate is not None:
            mutate(codes, scale, w)
        kdeq = O.e4m3_decode(codes) * scale[..., None].astype(np.float64)
        ik = torch.from_numpy(codes).to(DEV)
        iks = dev_f32(scale)
    else:
        kb = synth.normal_bf16((B, ik_ld, dI), 1.28, cfg, 23)
        if ties:
            kb[:, : n_cap // 2] = kb[:, :1]
        kdeq = synth.bf16_bits_to_f64(kb)
        ik = from_bits(kb)
        iks = None
    pos = np.array(positions, dtype=np.int64).reshape(B, Tq)
    idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=DEV)
    sc = torch.zeros((B, Tq, k), dtype=torch.float32, device=DEV)
    L.csa_index_topk(from_bits(q), from_bits(w), ik, iks, dev_i64(pos), n_cap=n_cap, m=m, k=k, topk_idx=idx,
                     topk_score=sc)
    torch.cuda.synchronize()
    gi, gs = idx.cpu().numpy(), sc.cpu().numpy()
    band = 0
    for b in range(B):
        for t in range(Tq):
            nv = min(pos[b, t] // m, n_cap)
            # many rows take the prefill scorer (its |a| / linear evaluation, see index_oracle_row)
            ref, bound = index_oracle_row(q[b, t], w[b, t], kdeq[b, :nv], fp8, split=fp8 and B * Tq >= 64)
            band += check_topk_row(gi[b, t], ref, k, bound)
            sel = gi[b, t][gi[b, t] >= 0]
            # scores agree within the fp32 accumulation bound of each selected entry
            assert np.all(np.abs(gs[b, t, : sel.size] - ref[sel]) <= bound[sel] + 1e-30)
            assert np.all(np.isneginf(gs[b, t, sel.size:]))
    return (band, gi) if return_idx else band


def test_index_topk_decode_fp8():
    # n_cap spans 3 score chunks and a ragged tail; rows with n_vis = 0, < k, == k, > k
    n_cap, k = 2600, 64
    pos = [0, 3, 100, 256, 257, 4 * 2600 + 9, 5000, 4 * 2600]
    band = _index_case(8, 1, n_cap, 64, 128, k, 4, True, pos, 31)
    assert band <= 2


def test_index_topk_workspace_left_zeroed_and_reusable():
    """One zero-filled workspace serves a sequence of calls of different shapes (decode rows, a
    many-row call, decode again): each call's selection equals a call on a fresh zeroed workspace
    (bit for bit), and after every call the workspace's leading state bytes are zero again."""
    shapes = [(8, 1, 20000, 512, 71), (3, 1, 9000, 256, 72), (1, 70, 5000, 128, 73), (5, 1, 30000, 1024, 74)]
    need = max(L.csa_index_topk_workspace(B, Tq, n, k) for B, Tq, n, k, _ in shapes)
    shared = L.workspace(need, zeroed=True)
    state = L.lib().csa_index_topk_state_bytes()
    assert 0 < state <= need
    for B, Tq, n_cap, k, cfg in shapes:
        print(f"shared workspace: B={B} Tq={Tq} n_cap={n_cap} k={k}", flush=True)
        q = from_bits(synth.normal_bf16((B, Tq, 64, 128), 1.28, cfg, 1))
        w = from_bits(synth.normal_bf16((B, Tq, 64), 1.28, cfg, 2))
        codes = torch.from_numpy(synth.fp8_codes((B, n_cap, 128), cfg, 3)).to(DEV)
        scale = dev_f32(synth.positive_scales((B, n_cap), cfg, 4))
        pos = 4 * n_cap - 2 * np.arange(B * Tq, dtype=np.int64).reshape(B, Tq) * (n_cap // (B * Tq + 1))
        outs = []
        for ws in (shared, None):
            idx = torch.full((B, Tq, k), -7, dtype=torch.int32, device=DEV)
            L.csa_index_topk(q, w, codes, scale, dev_i64(pos), n_cap=n_cap, m=4, k=k, topk_idx=idx, ws=ws)
            outs.append(idx)
        torch.cuda.synchronize()
        assert torch.equal(outs[0], outs[1])
        assert int(shared[:state].count_nonzero()) == 0


@pytest.mark.parametrize("fp8,H_I,dI", [(True, 8, 128), (True, 40, 128), (False, 40, 128), (False, 40, 64)])
def test_index_topk_decode_head_blocks_ragged(fp8, H_I, dI):
    # decode scoring with padded head blocks (8 -> 16, 40 -> 48 heads) and chunks that end inside a
    # 64-entry group: rows with n_vis = 0, < k, == k, ragged and at capacity
    n_cap, k = 3001, 96
    pos = [0, 5, 4 * 96, 4 * 1023 + 3, 4 * 3001, 4 * 2999 + 1]
    band = _index_case(6, 1, n_cap, H_I, dI, k, 4, fp8, pos, 41 + H_I + dI)
    assert band <= 2


def test_index_topk_prefill_fp8_rowwise():
    Tq, n_cap, k = 80, 1500, 100
    pos = list(range(4 * 1500 - 79, 4 * 1500 + 1)) + list(range(0, 800, 10))
    band = _index_case(2, Tq, n_cap, 64, 128, k, 4, True, pos, 32)
    assert band <= 4


@pytest.mark.parametrize("H_I,Tq,n_cap", [(8, 33, 1500), (16, 37, 2500), (40, 50, 1100), (64, 35, 5000)])
def test_index_topk_prefill_fp8_head_blocks_ragged(H_I, Tq, n_cap):
    # fp8 prefill scoring with 1 (8 heads padded to 16, and 16) / 3 / 4 blocks of 16 heads; Tq not a
    # multiple of 4 (the last group of 4 queries is partly empty); batch row 0 at the end of the
    # cache, row 1 spread from empty (t < m) through partial visibility to full; n_cap spanning
    # several 1024-entry chunks + a tail
    k = 96
    full = list(range(4 * n_cap - Tq + 1, 4 * n_cap + 1))
    spread = [int(x) for x in np.linspace(0, 4 * n_cap + 20, Tq)]
    band = _index_case(2, Tq, n_cap, H_I, 128, k, 4, True, full + spread, 36 + H_I)
    assert band <= 4


@pytest.mark.parametrize("B,Tq,H_I,dI,fp8", [(3, 700, 16, 128, True), (2, 1100, 8, 64, False)])
def test_index_topk_prefill_query_batches(B, Tq, H_I, dI, fp8):
    # many rows whose buffers exceed 64 MiB are scored and selected in batches of query positions
    # (B * batch <= 768 rows of buffers): 3 x 700 rows of 3008 entries runs batches of 256, 256 and
    # 188 positions, 2 x 1100 of 384, 384 and 332, so batch edges, a short last batch and every batch
    # row are covered, with rows from empty to full
    n_cap, k = 3000, 64
    assert L.csa_index_topk_workspace(B, Tq, n_cap, k) < B * Tq * 3008 * 12   # less than one batch would need
    pos = []
    for b in range(B):
        if b % 2 == 0:
            pos += [int(x) for x in np.linspace(0, 4 * n_cap + 30, Tq)]
        else:
            pos += list(range(4 * n_cap - Tq + 1, 4 * n_cap + 1))
    band = _index_case(B, Tq, n_cap, H_I, dI, k, 4, fp8, pos, 45 + B)
    assert band <= 2 * B * Tq // 100 + 4


def test_index_topk_prefill_long_rows_sampled_threshold():
    # rows long enough for the sampled threshold (n_vis >= 8192 and >= 8 k) next to shorter ones
    n_cap, k, Tq = 12000, 128, 64
    pos = [int(x) for x in np.linspace(4 * 6000, 4 * n_cap + 40, Tq)]
    band = _index_case(1, Tq, n_cap, 64, 128, k, 4, True, pos, 37)
    assert band <= 4


def test_index_topk_prefill_sampled_threshold_falls_back():
    # Only the entries a 32-entry-run sample reads score above zero, all distinct: the sample's
    # threshold then passes fewer than k entries and the row must take the full selection.
    n_cap, k, Tq = 32768, 256, 64
    sampled = (np.arange(n_cap) % 512) < 32

    def mutate(codes, scale, w):
        codes[:, :n_cap][:, ~sampled] = 0
        codes[:, :n_cap][:, sampled] = codes[:, :1]
        scale[:, :n_cap] = (np.float32(2.0) + np.arange(n_cap, dtype=np.float32) / np.float32(n_cap)) / np.float32(448.0)
        w &= np.uint16(0x7FFF)                  # positive head weights: every sampled score > 0

    band = _index_case(1, Tq, n_cap, 64, 128, k, 4, True, [4 * n_cap] * Tq, 38, mutate=mutate)
    assert band <= 4


def test_index_topk_prefill_sampled_threshold_top_ties():
    # Half of each long row is one repeated key with a scale 64x the others' and positive head
    # weights, so it scores on top: the sampled threshold keeps ~6000 tied candidates (more than the
    # LDS array holds, so the candidate pass runs again into global memory and the digit passes read
    # them from there) and the k winners must be
    # the lowest indices among the ties.  (The oracle's fp64 matrix products may round equal rows
    # differently by position, so its own order among the ties is not the reference here: the tie
    # rule is, and the within-bound check of every row still runs.)
    n_cap, k, Tq = 12000, 128, 64

    def mutate(codes, scale, w):
        codes[:, : n_cap // 2] = codes[:, :1]
        scale[:, : n_cap // 2] = scale[:, :1] * np.float32(64.0)
        w &= np.uint16(0x7FFF)

    pos = [int(x) for x in np.linspace(4 * 9000, 4 * n_cap, Tq)]
    _, gi = _index_case(1, Tq, n_cap, 64, 128, k, 4, True, pos, 39, mutate=mutate, return_idx=True)
    np.testing.assert_array_equal(gi[0], np.broadcast_to(np.arange(k, dtype=np.int32), (Tq, k)))


def test_index_topk_bf16_small_heads():
    # the prefill-2k shape family: 8 heads x 64 dims, bf16 keys, top-k 128
    Tq, n_cap, k = 70, 512, 128
    pos = list(range(2048 - Tq, 2048))
    _index_case(1, Tq, n_cap, 8, 64, k, 4, False, pos, 33)


def _short_row_positions(Tq, n_cap, k):
    # n_vis = 0, 1, k - 1, k, k + 1, k + 2, capacity - 1 and capacity, the rest spread between
    nvs = [0, 1, k - 1, k, k + 1, k + 2, n_cap - 1, n_cap]
    nvs += [int(x) for x in np.linspace(0, n_cap, Tq - len(nvs))]
    return [4 * v + (i % 4) for i, v in enumerate(nvs)]


@pytest.mark.parametrize("fp8,n_cap,k,ties", [(True, 1024, 100, False), (False, 1000, 256, False),
                                              (True, 700, 512, True), (False, 1024, 1000, True)])
def test_index_topk_prefill_short_rows(fp8, n_cap, k, ties):
    # rows of at most 1024 visible entries take one wave each: trivial rows (n_vis <= k), one entry
    # over k, and full rows whose last lanes lie past the row; with half the keys tied, the ties at
    # the k-th key go to the lower index
    Tq = 72
    H_I, dI = (64, 128) if fp8 else (8, 64)
    band = _index_case(1, Tq, n_cap, H_I, dI, k, 4, fp8, _short_row_positions(Tq, n_cap, k), 57 + k, ties=ties)
    assert band <= 4


@pytest.mark.parametrize("fp8,k", [(True, 100), (False, 256), (True, 1000)])
def test_index_topk_short_rows_wave_path_matches_workgroup_path(fp8, k):
    """The same rows (n_vis <= 1024) selected by the one-wave path (capacity 1024) and by the
    workgroup path (capacity 1088): the same scores and the same tie rule give identical indices
    and scores, with and without a tied half of the keys."""
    Tq, cfg = 72, 58 + k
    H_I, dI = (64, 128) if fp8 else (8, 64)
    ik_ld = 1088 + 5
    q = from_bits(synth.normal_bf16((1, Tq, H_I, dI), 1.28, cfg, 1))
    w = from_bits(synth.normal_bf16((1, Tq, H_I), 1.28, cfg, 2))
    pos = dev_i64(np.array(_short_row_positions(Tq, 1024, k), dtype=np.int64).reshape(1, Tq))
    for ties in (False, True):
        if fp8:
            codes = synth.fp8_codes((1, ik_ld, dI), cfg, 3)
            scale = synth.positive_scales((1, ik_ld), cfg, 4)
            if ties:
                codes[:, :512] = codes[:, :1]
                scale[:, :512] = scale[:, :1]
            ik, iks = torch.from_numpy(codes).to(DEV), dev_f32(scale)
        else:
            kb = synth.normal_bf16((1, ik_ld, dI), 1.28, cfg, 3)
            if ties:
                kb[:, :512] = kb[:, :1]
            ik, iks = from_bits(kb), None
        res = []
        for n_cap in (1024, 1088):
            idx = torch.full((1, Tq, k), -7, dtype=torch.int32, device=DEV)
            sc = torch.zeros((1, Tq, k), dtype=torch.float32, device=DEV)
            L.csa_index_topk(q, w, ik, iks, pos, n_cap=n_cap, m=4, k=k, topk_idx=idx, topk_score=sc)
            res.append((idx, sc))
        torch.cuda.synchronize()
        assert torch.equal(res[0][0], res[1][0]), f"ties={ties}: indices differ"
        assert torch.equal(res[0][1], res[1][1]), f"ties={ties}: scores differ"


@pytest.mark.parametrize("fp8,n_cap", [(True, 3000), (False, 3000), (True, 12000)])
def test_index_topk_exact_ties_go_to_lower_index(fp8, n_cap):
    # half the keys identical: the tied block fills the threshold bin (12000: more candidates than
    # the final kernel stages in LDS, so its passes read the kept list from global memory)
    k = 40
    _index_case(2, 1, n_cap, 16 if fp8 else 8, 128 if fp8 else 64, k, 4, fp8, [4 * n_cap, 3 * n_cap], 34, ties=True)


def test_index_topk_all_equal_scores():
    """Identical keys: every score ties, the k lowest indices must be returned."""
    B, n_cap, k = 2, 5000, 77
    q = synth.normal_bf16((B, 1, 64, 128), 1.28, 35, 1)
    w = synth.normal_bf16((B, 1, 64), 1.28, 35, 2)
    codes = np.repeat(synth.fp8_codes((B, 1, 128), 35, 3), n_cap, axis=1)
    scale = np.full((B, n_cap), 0.01, dtype=np.float32)
    idx = torch.empty((B, 1, k), dtype=torch.int32, device=DEV)
    L.csa_index_topk(from_bits(q), from_bits(w), torch.from_numpy(codes).to(DEV), dev_f32(scale),
                     dev_i64(np.array([[4 * n_cap], [4 * 3000 + 3]])), n_cap=n_cap, m=4, k=k, topk_idx=idx)
    got = idx.cpu().numpy()
    np.testing.assert_array_equal(got[0, 0], np.arange(k))
    np.testing.assert_array_equal(got[1, 0], np.arange(k))


# ----------------------------------------------------------------------------------- attention
def _attend_case(kind, B, Tq, H, k, n_cap, m, W, ring_cap, positions, cfg, sink_inf=False, rope_offset=0,
                 block_scale=None, gamma_scale=1.0, eps=1e-6, q_signs=False, kv8=False, no_ring=False):
    q = synth.normal_bf16((B, Tq, H, 512), 1.28, cfg, 41)
    if q_signs:   # entries +-1: with eps = 0 the normalised query is gamma * q, exact in bf16
        q = synth.f32_to_bf16_bits(np.where(synth.bf16_bits_to_f64(q) >= 0, 1.0, -1.0).astype(np.float32))
    gq = synth.f32_to_bf16_bits(gamma_scale * (0.5 + synth.rng(cfg, 42).random(512, dtype=np.float32)))
    kv_ld = n_cap + 3
    cache = synth.normal_bf16((B, kv_ld, 512), 1.0, cfg, 43)
    if block_scale is not None:
        # entries in alternating blocks of 32 scaled by (small, big): the logit range jumps by far more
        # than the lazy-rescale margin from one tile to the next
        small, big = block_scale
        f = np.where((np.arange(kv_ld) // 32) % 2 == 0, small, big)[None, :, None]
        cache = synth.f32_to_bf16_bits((synth.bf16_bits_to_f64(cache) * f).astype(np.float32))
    pos = np.array(positions, dtype=np.int64).reshape(B, Tq)
    max_t = int(pos.max())
    win_ld = ring_cap if ring_cap else max_t + 1
    win_tok = synth.normal_bf16((B, win_ld, 512), 1.0, cfg, 44)   # row j % ring_cap holds token j
    sink = np.full(H, -np.inf, np.float32) if sink_inf else synth.normal_f32((H,), 1.0, cfg, 45)
    out = torch.zeros((B, Tq, H, 512), dtype=torch.bfloat16, device=DEV)
    scale = 1.0 / math.sqrt(512)
    cache64 = synth.bf16_bits_to_f64(cache)
    win64 = synth.bf16_bits_to_f64(win_tok)
    kv_dev, win_dev, extra = from_bits(cache), from_bits(win_tok), {}
    if kv8:   # fp8 K=V storage: codes and row scales from the oracle's quantiser (fp32 decisions)
        ccodes, csc, cache64 = O.fp8_quantize_rows(cache64, kernel_fp32=True)
        wcodes, wsc, win64 = O.fp8_quantize_rows(win64, kernel_fp32=True)
        kv_dev, win_dev = torch.from_numpy(ccodes).to(DEV), torch.from_numpy(wcodes).to(DEV)
        extra = dict(kv_scale=dev_f32(csc), win_scale=dev_f32(wsc))
    if no_ring:   # window = 0 and no ring at all (NULL codes / rows and scales)
        assert W == 0
        win_dev = None
        if kv8:
            extra["win_scale"] = None
    if kind == "csa":
        g = synth.rng(cfg, 46)
        topk = -np.ones((B, Tq, k), dtype=np.int32)
        for b in range(B):
            for t in range(Tq):
                nv = min(pos[b, t] // m, n_cap)
                sel = np.sort(g.choice(nv, size=min(k, nv), replace=False)) if nv else np.zeros(0, int)
                topk[b, t, : sel.size] = sel
        L.csa_attend(from_bits(q), from_bits(gq), kv_dev, torch.from_numpy(topk).to(DEV),
                     win_dev, dev_f32(sink), dev_i64(pos), window=W, ring_cap=ring_cap, out=out,
                     rope_offset=rope_offset, eps=eps, **extra)
    else:
        L.hca_attend(from_bits(q), from_bits(gq), kv_dev, win_dev, dev_f32(sink), dev_i64(pos),
                     n_cap=n_cap, m=m, window=W, ring_cap=ring_cap, out=out, rope_offset=rope_offset, eps=eps,
                     **extra)
    torch.cuda.synchronize()
    got = to_np_bf16(out)
    g64 = synth.bf16_bits_to_f64(gq)
    worst = (0.0, 0.0)
    for b in range(B):
        for t in range(Tq):
            tt = int(pos[b, t])
            nv = min(tt // m, n_cap)
            keys = [cache64[b, s] for s in (topk[b, t][topk[b, t] >= 0] if kind == "csa" else range(nv))]
            for j in range(max(0, tt - W + 1), tt + 1):
                keys.append(win64[b, j % ring_cap if ring_cap else j])
            K = np.stack(keys) if keys else np.zeros((0, 512))
            ref = O.attend_one(synth.bf16_bits_to_f64(q[b, t]), g64, K, sink.astype(np.float64), tt, scale,
                               eps, 10000.0, rope_offset)
            ma, rl = assert_close(got[b, t], ref, f"{kind} b={b} t={tt}")
            worst = (max(worst[0], ma), max(worst[1], rl))
    return worst


@pytest.mark.parametrize("H", [64, 8, 32])
def test_csa_attend_parity(H):
    # k + W keys spread over several tiles; some rows padded with -1 (n_vis < k)
    pos = [4 * 900 + 2, 37, 4 * 500, 130]
    _attend_case("csa", 2, 2, H, 200, 900, 4, 128, 256, pos, 51 + H)


def test_csa_attend_linear_window_and_minus_inf_sink():
    _attend_case("csa", 1, 3, 64, 64, 300, 4, 20, 0, [1199, 1000, 5], 52, sink_inf=True)


@pytest.mark.parametrize("n_cap,H", [(700, 64), (3000, 64), (60, 16)])
def test_hca_attend_parity(n_cap, H):
    # dense over all visible entries: many splits (3000) and a single split (60)
    pos = [128 * n_cap + 5, 128 * n_cap // 2 + 127, 0]
    _attend_case("hca", 3, 1, H, 0, n_cap, 128, 128, 128, pos, 53 + n_cap)


def test_hca_attend_running_max_jumps_rescale_accumulators():
    # Every split sees a tile of tiny logits followed by one of large logits (a 6x query gamma, keys
    # scaled 0.02 / 1 in alternating blocks of 32), so the running max moves by far more than the
    # kernel's lazy margin and the accumulated output is rescaled mid-split.  Logits this large would
    # turn the bf16 rounding of the normalised query into percent-level output differences, so the
    # query is made exactly representable: entries +-1, eps = 0 and position 0 after the offset
    # (the rotation is the identity), which leaves qhat = gamma * q.
    t = 128 * 700 + 5
    _attend_case("hca", 2, 1, 64, 0, 700, 128, 128, 128, [t, t], 56, block_scale=(0.02, 1.0), gamma_scale=6.0,
                 eps=0.0, q_signs=True, rope_offset=-t)


@pytest.mark.parametrize("kind,H", [("csa", 64), ("csa", 8), ("hca", 64), ("hca", 16)])
def test_attend_fp8_kv_parity(kind, H):
    """fp8 K=V storage (codes + one scale per row, cache and ring) against the oracle on the same
    dequantised keys: the bf16 bar (the codes are converted exactly; only the scales enter the
    logits and the PV weights)."""
    if kind == "csa":
        _attend_case("csa", 2, 2, H, 200, 900, 4, 128, 256, [4 * 900 + 2, 37, 4 * 500, 130], 151 + H, kv8=True)
    else:
        n_cap = 700 if H == 64 else 60
        _attend_case("hca", 3, 1, H, 0, n_cap, 128, 128, 128, [128 * n_cap + 5, 128 * n_cap // 2 + 127, 0],
                     153 + n_cap, kv8=True)


@pytest.mark.parametrize("kv8", [True, False])
def test_attend_without_window_ring(kv8):
    """window = 0 with no ring passed (NULL rows, NULL scales): CSA with k = 300 (a ragged last tile)
    and rows padded with -1, and HCA with a query at t = 0 and one at t < m', whose key splits are
    all empty (their outputs are 0: no key, only the sink)."""
    _attend_case("csa", 2, 1, 64, 300, 900, 4, 0, 0, [4 * 900 + 2, 4 * 200 + 1], 171, kv8=kv8, no_ring=True)
    _attend_case("hca", 3, 1, 64, 0, 700, 128, 0, 0, [128 * 700 + 5, 0, 100], 172, kv8=kv8, no_ring=True)


def test_hca_attend_fp8_kv_running_max_jumps():
    t = 128 * 700 + 5
    _attend_case("hca", 2, 1, 64, 0, 700, 128, 128, 128, [t, t], 156, block_scale=(0.02, 1.0), gamma_scale=6.0,
                 eps=0.0, q_signs=True, rope_offset=-t, kv8=True)


def test_csa_attend_list_entries_past_the_cache_are_missing_keys():
    """A selection slot holding an index past the cache (a slot nobody filled) is no key, exactly
    like -1: the outputs are bitwise equal (the kernel's own bound, no read past the cache)."""
    B, H, k, n_cap, W, ring = 1, 64, 64, 300, 128, 256
    t = 4 * n_cap
    q = synth.normal_bf16((B, 1, H, 512), 1.28, 161, 1)
    gq = synth.f32_to_bf16_bits(np.ones(512, np.float32))
    cache = synth.normal_bf16((B, n_cap, 512), 1.0, 161, 2)
    win = synth.normal_bf16((B, ring, 512), 1.0, 161, 3)
    sink = synth.normal_f32((H,), 1.0, 161, 4)
    sel = np.sort(synth.rng(161, 5).choice(n_cap, k, replace=False)).astype(np.int32)
    bad, none = sel.copy(), sel.copy()
    bad[[3, 17, 40]] = [n_cap, n_cap + 12345, 2 ** 30]
    none[[3, 17, 40]] = -1
    outs = []
    for lst in (bad, none):
        out = torch.zeros((B, 1, H, 512), dtype=torch.bfloat16, device=DEV)
        L.csa_attend(from_bits(q), from_bits(gq), from_bits(cache), torch.from_numpy(lst.reshape(B, 1, k)).to(DEV),
                     from_bits(win), dev_f32(sink), dev_i64(np.array([[t]])), window=W, ring_cap=ring, out=out)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


@pytest.mark.parametrize("H,B,Tq,kv8,ring", [(8, 1, 130, False, 0), (16, 2, 67, False, 512), (32, 1, 129, True, 0),
                                         (8, 2, 70, True, 512), (8, 1, 128, False, 64)])
def test_csa_attend_row_blocks(H, B, Tq, kv8, ring):
    # many query rows over a small cache (at most 2048 entries) with 8, 16 or 32 heads: a workgroup
    # takes 64 / H consecutive rows of one sequence (ragged last blocks) and attends to the union of
    # their lists and windows, each row keeping only its own keys.  Positions are spread (sorted
    # random), so the block's window range holds tokens no row uses; with the 64-token ring that
    # range is longer than the ring.  Early rows have fewer visible entries than k (-1 slots).
    n_cap, k, W = 300, 64, 64
    pos = np.sort(synth.rng(190 + H, 7).integers(20, 4 * n_cap + 50, size=(B, Tq)), axis=1)
    if ring == 64:
        pos = np.arange(Tq).reshape(1, Tq) * 9 + 40
    _attend_case("csa", B, Tq, H, k, n_cap, 4, W, ring, pos.ravel().tolist(), 191 + H, kv8=kv8)


def test_csa_attend_row_blocks_entries_past_the_cache_are_missing_keys():
    """Row blocks: list slots holding an index past the cache are no key, exactly like -1."""
    B, Tq, H, k, n_cap, W, ring = 1, 128, 8, 64, 300, 128, 512
    q = synth.normal_bf16((B, Tq, H, 512), 1.28, 171, 1)
    gq = synth.f32_to_bf16_bits(np.ones(512, np.float32))
    cache = synth.normal_bf16((B, n_cap, 512), 1.0, 171, 2)
    win = synth.normal_bf16((B, ring, 512), 1.0, 171, 3)
    sink = synth.normal_f32((H,), 1.0, 171, 4)
    g = synth.rng(171, 5)
    sel = np.stack([np.sort(g.choice(n_cap, k, replace=False)) for _ in range(Tq)]).astype(np.int32)
    bad, none = sel.copy(), sel.copy()
    bad[::3, [3, 17, 40]] = [n_cap, n_cap + 12345, 2 ** 30]
    none[::3, [3, 17, 40]] = -1
    pos = np.arange(4 * n_cap, 4 * n_cap + Tq).reshape(B, Tq)
    outs = []
    for lst in (bad, none):
        out = torch.zeros((B, Tq, H, 512), dtype=torch.bfloat16, device=DEV)
        L.csa_attend(from_bits(q), from_bits(gq), from_bits(cache), torch.from_numpy(lst.reshape(B, Tq, k)).to(DEV),
                     from_bits(win), dev_f32(sink), dev_i64(pos), window=W, ring_cap=ring, out=out)
        outs.append(out)
    torch.cuda.synchronize()
    assert torch.equal(outs[0], outs[1])


def test_kv_quantize_fp8_bit_exact():
    """The device quantiser of K=V rows against the oracle's (fp32 decisions): codes and scales
    identical, on Gaussian rows at several magnitudes, an all-zero row, rows with one huge value,
    and rows that put many values exactly on E4M3FN rounding ties."""
    rows = synth.normal_bf16((300, 512), 1.0, 160, 1)
    f = synth.bf16_bits_to_f64(rows)
    f[:100] *= 37.0
    f[100:150] *= 1e-3
    f[150] = 0.0
    f[151] = 0.0
    f[151, 7] = -3e4
    ties = np.array([448.0, 9.0 / 16, 17.0 / 32, 0.75 + 1 / 32, 2.0 ** -9 * 1.5], dtype=np.float64)
    f[152:160] = np.resize(np.concatenate([ties, -ties]), (8, 512))
    bits = synth.f32_to_bf16_bits(f.astype(np.float32))
    codes = torch.empty((300, 512), dtype=torch.uint8, device=DEV)
    scales = torch.empty((300,), dtype=torch.float32, device=DEV)
    L.kv_quantize_fp8(from_bits(bits), codes=codes, scales=scales)
    torch.cuda.synchronize()
    rc, rs, _ = O.fp8_quantize_rows(synth.bf16_bits_to_f64(bits), kernel_fp32=True)
    assert np.array_equal(codes.cpu().numpy(), rc)
    assert np.array_equal(scales.cpu().numpy(), rs.astype(np.float32))


def test_hca_attend_single_split_finishes_in_kernel():
    # 30 entries + 32 window keys = 2 tiles: one split, the attention kernel writes the output itself
    assert L.attend_workspace(2, 1, 16, 62) == 256
    _attend_case("hca", 2, 1, 16, 0, 30, 128, 32, 64, [128 * 30 + 1, 128 * 15], 55)


def test_hca_attend_prefill_rows_with_rope_offset():
    pos = list(range(4000, 4000 + 40))
    _attend_case("hca", 1, 40, 64, 0, 40, 128, 128, 0, pos, 54, rope_offset=12345)


@pytest.mark.parametrize("kind,H", [("csa", 40), ("hca", 40), ("hca", 24)])
def test_attend_head_blocks_of_padding_only(kind, H):
    # head counts that leave a workgroup's last block(s) of 16 head slots without a real head: CSA
    # decode with 40 heads in two halves of 32 slots (heads 32..39 in the second), HCA with 40 heads
    # in 64 slots (blocks 0..2 hold heads) and 24 heads in 32 slots
    if kind == "csa":
        _attend_case("csa", 2, 2, H, 200, 900, 4, 128, 256, [4 * 900 + 2, 37, 4 * 500, 130], 181 + H)
    else:
        _attend_case("hca", 3, 1, H, 0, 700, 128, 128, 128, [128 * 700 + 5, 128 * 350 + 127, 0], 183 + H)


@pytest.mark.parametrize("H", [40, 8])
def test_csa_attend_many_rows_padding_head_blocks(H):
    # 130 query rows (the many-row layout, one split per row) with 40 heads (64 slots, one block of
    # padding) and 8 heads (32 slots, one block holds all of them)
    pos = [1000 + 3 * i for i in range(130)]
    _attend_case("csa", 1, 130, H, 64, 300, 4, 64, 0, pos, 185 + H)


# ----------------------------------------------------------------------------------- projection
# M = 8: the decode GEMV; 3 and 37: the row-block kernel; 64, 130 and 300 rows: the tiled prefill GEMM
# (one and several 128-row blocks, ragged last block, one group and eight); 600 rows: the 256 x 256
# blocks (two whole row blocks and a ragged one, two groups of 256 features, then one group)
@pytest.mark.parametrize("M,H,g,d_g,d", [(8, 64, 8, 1024, 4096), (3, 16, 2, 64, 96), (37, 8, 1, 32, 48),
                                         (64, 16, 2, 128, 256), (130, 8, 1, 128, 384), (300, 64, 8, 1024, 4096),
                                         (600, 16, 2, 256, 512)])
def test_grouped_out_proj_parity(M, H, g, d_g, d):
    cfg = 60 + M
    o = synth.normal_bf16((M, H * 512), 0.3, cfg, 1)
    wg = synth.normal_bf16((g, d_g, H * 512 // g), 0.02, cfg, 2)
    wo = synth.normal_bf16((d, g * d_g), 0.02, cfg, 3)
    y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    L.grouped_out_proj(from_bits(o), from_bits(wg), from_bits(wo), H=H, y=y)
    torch.cuda.synchronize()
    _, ref = O.grouped_out_proj(synth.bf16_bits_to_f64(o), synth.bf16_bits_to_f64(wg), synth.bf16_bits_to_f64(wo))
    assert_close(to_np_bf16(y), ref, "grouped out-proj")
