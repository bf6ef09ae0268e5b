"""Pins of the CPU oracle against what the pages and the mathematics fix (no GPU).

Each test checks the oracle against something other than itself: closed forms,
invariants the pages state, textbook/library routines (numpy complex products,
scipy softmax/block_diag, torch float64 attention, torch's E4M3FN cast) and
brute force on tiny inputs.
"""
import math
import os

import numpy as np
import pytest
import scipy.linalg
import scipy.special
import torch

import oracle as O
import synth
from synth import configs

GOLD = os.path.join(os.path.dirname(__file__), "golden")
RNG = np.random.default_rng(1234)


def randn(*shape, std=1.0):
    return RNG.standard_normal(shape) * std


# ------------------------------------------------------------------------------- constants
def test_page_constants_match_workloads():
    vals = {}
    for line in open(os.path.join(GOLD, "page_constants.txt")):
        if line.startswith("#") or not line.strip():
            continue
        name, v = line.split()[:2]
        vals[name] = int(v)
    assert O.C_HEAD == vals["head_dim"] and O.ROPE_DIMS == vals["rope_dims"]
    w3 = configs.CONFIGS["csa_decode_128k"]
    assert (w3.m, w3.m_hca, w3.H_I, w3.d_I, w3.k, w3.W) == (
        vals["m_csa"], vals["m_hca"], vals["indexer_heads"], vals["indexer_dim"], vals["topk_flash"],
        vals["window"])
    assert configs.CONFIGS["hybrid4_decode_1m"].k == vals["topk_1m"] == configs.CONFIGS["csa_chunked_prefill_1m"].k


# ------------------------------------------------------------------------------- RMSNorm
def test_rmsnorm_unit_rms_and_scale_invariance():
    x = randn(7, 512, std=3.0)
    g = 0.5 + RNG.random(512)
    y = O.rmsnorm(x, g, 0.0)
    np.testing.assert_allclose(np.sqrt(np.mean((y / g) ** 2, axis=-1)), 1.0, rtol=1e-12)
    np.testing.assert_allclose(O.rmsnorm(5.0 * x, g, 0.0), y, rtol=1e-12)
    # eps enters under the root: a zero vector stays zero, a tiny one is damped
    assert np.all(O.rmsnorm(np.zeros(512), g, 1e-6) == 0)


def test_rmsnorm_eps_under_the_root_closed_form():
    """A constant vector c: RMSNorm gives gamma * c / sqrt(c^2 + eps).  At c = 1e-3, eps = 1e-6 this is
    gamma / sqrt(2): eps added outside the root (0.999), left out (1) or a sum instead of a mean
    (1/sqrt(512)) all fail."""
    g = 0.5 + RNG.random(512)
    for c, eps in ((1e-3, 1e-6), (2.0, 0.5), (-3.0, 1e-6), (0.25, 0.0)):
        got = O.rmsnorm(np.full(512, c), g, eps)
        np.testing.assert_allclose(got, g * c / math.sqrt(c * c + eps), rtol=1e-14)
    np.testing.assert_allclose(O.rmsnorm(np.full(512, 1e-3), np.ones(512), 1e-6), 2 ** -0.5, rtol=1e-12)


# ------------------------------------------------------------------------------- RoPE
def test_rope_matches_complex_rotation():
    x = randn(512)
    p = 987.0
    y = O.rope(x, p)
    np.testing.assert_array_equal(y[:448], x[:448])
    z = x[448::2] + 1j * x[449::2]
    j = np.arange(32)
    zr = z * np.exp(1j * p * 10000.0 ** (-j / 32.0))
    np.testing.assert_allclose(y[448::2], zr.real, atol=1e-12)
    np.testing.assert_allclose(y[449::2], zr.imag, atol=1e-12)


def test_rope_group_and_relative_properties():
    x, k = randn(512), randn(512)
    np.testing.assert_allclose(O.rope(x, 0), x, atol=0)
    np.testing.assert_allclose(O.rope(O.rope(x, 37), 1000.5), O.rope(x, 1037.5), atol=1e-9)
    np.testing.assert_allclose(np.linalg.norm(O.rope(x, 123456)), np.linalg.norm(x), rtol=1e-12)
    # only relative position survives in a dot product
    a = np.dot(O.rope(x, 500), O.rope(k, 200))
    b = np.dot(O.rope(x, 300 + 1e6), O.rope(k, 1e6))
    assert abs(a - b) < 1e-8 * max(1, abs(a))
    # angles: j = 0 turns by p radians, j = 16 by p/100
    ang = O.rope_angles(50.0)
    assert ang[0] == 50.0 and abs(ang[16] - 0.5) < 1e-15


# ------------------------------------------------------------------------------- pooling
def test_pool_closed_forms():
    x = randn(16, 8)
    s = randn(16)
    np.testing.assert_allclose(O.pool(x, s, 1, 0), x, atol=1e-15)                  # m = 1: identity
    e = O.pool(x, np.zeros(16), 4, 0)
    np.testing.assert_allclose(e, x.reshape(4, 4, 8).mean(axis=1), atol=1e-15)     # equal logits: mean
    s2 = np.zeros(16)
    s2[6] = 60.0
    e2 = O.pool(x, s2, 4, 4)                                                       # +60 logit dominates
    np.testing.assert_allclose(e2[1], x[6], atol=1e-20 + 1e-24)
    np.testing.assert_allclose(e2[2], x[6], atol=1e-20)                            # overlap reaches back
    assert not np.allclose(e2[3], x[6])


def test_pool_brute_force_overlap_windows():
    m, ov, T = 4, 4, 14
    x, s = randn(T, 5), randn(T)
    e = O.pool(x, s, m, ov)
    assert e.shape == (T // m, 5)
    for i in range(T // m):
        toks = [j for j in range(T) if i * m - ov <= j < (i + 1) * m]            # the reading, spelled out
        w = scipy.special.softmax(s[toks])
        np.testing.assert_allclose(e[i], (w[:, None] * x[toks]).sum(0), atol=1e-13)
    assert [len(range(*O.block_span(i, m, ov))) for i in range(3)] == [4, 8, 8]


def test_compress_kv_norm_then_rope_at_block_end():
    x, s = randn(12, 512), randn(12)
    g = np.ones(512)
    ent = O.compress_kv(x, s, 4, 4, g, eps=0.0)
    e = O.pool(x, s, 4, 4)
    for i in range(3):
        back = O.rope(ent[i], -(4 * i + 3))          # un-rotate from the block's last token
        np.testing.assert_allclose(back, O.rmsnorm(e[i], g, 0.0), atol=1e-12)
        np.testing.assert_allclose(np.sqrt(np.mean(ent[i] ** 2)), 1.0, rtol=1e-12)


# ------------------------------------------------------------------------------- fp8 E4M3FN
def test_e4m3_anchor_values():
    for line in open(os.path.join(GOLD, "e4m3fn_anchors.txt")):
        if line.startswith("#") or not line.strip():
            continue
        code, val = line.split()
        assert O.e4m3_value(int(code, 16)) == float(val), code
    assert math.isnan(O.e4m3_value(0x7F)) and math.isnan(O.e4m3_value(0xFF))


def test_e4m3_roundtrip_all_finite_codes():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    vals = np.array([O.e4m3_value(c) for c in codes])
    back = O.e4m3_encode(vals)
    # -0 (0x80) encodes back to +0; every other code is exact
    ok = (back == codes) | ((codes == 0x80) & (back == 0))
    assert ok.all()
    np.testing.assert_array_equal(O.e4m3_decode(codes), vals)


def test_e4m3_encode_exhaustive_bf16_against_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    v = synth.bf16_bits_to_f32(bits)
    fin = np.isfinite(v) & (np.abs(v) <= 448.0)
    v = v[fin]
    ours = O.e4m3_encode(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    # torch keeps the sign of zero; compare values
    np.testing.assert_array_equal(O.e4m3_decode(ours), O.e4m3_decode(ref))
    # saturation above the largest finite value
    assert (O.e4m3_encode(np.array([449.0, 1e9, -1e9])) == np.array([0x7E, 0x7E, 0xFE])).all()


def test_e4m3_nearest_and_ties_to_even():
    tab = O.e4m3_table()
    mids = (tab[1:] + tab[:-1]) / 2
    codes = O.e4m3_encode(mids)
    lower = np.arange(126)
    expect = np.where(lower % 2 == 0, lower, lower + 1)
    np.testing.assert_array_equal(codes, expect)
    x = RNG.random(10000) * 448
    c = O.e4m3_encode(x)
    err = np.abs(O.e4m3_decode(c) - x)
    nearest = np.min(np.abs(tab[None, :] - x[:, None]), axis=1)
    np.testing.assert_array_equal(err, nearest)


def test_fp8_row_quant_scales_absmax_to_448():
    v = randn(5, 128, std=1.3)
    codes, s, deq = O.fp8_quantize_rows(v)
    amax = np.abs(v).max(1)
    np.testing.assert_allclose(s, amax / 448.0)
    assert (np.abs(O.e4m3_decode(codes)).max(1) == 448.0).all()
    assert (np.abs(deq - v) <= np.abs(v) * 2.0 ** -4 + s[:, None] * 2.0 ** -10).all()
    c32, s32, _ = O.fp8_quantize_rows(v, kernel_fp32=True)
    assert (np.abs(c32.astype(int) - codes.astype(int)) <= 1).all()     # fp32 path differs at most one code
    zc, zs, zd = O.fp8_quantize_rows(np.zeros((1, 8)))
    assert zs[0] == 1.0 and (zd == 0).all()


def _torch_fp32_route(v):
    """An independent route to the fp32-decision row quantiser: torch float32 absmax, float32
    division of it by 448 (1 for an all-zero row), float32 division of every element by that scale,
    then torch's own E4M3FN cast (round to nearest, ties to even).  torch keeps the sign of a value
    that rounds to zero (0x80); the quantiser writes +0 there, so 0x80 is compared as 0x00."""
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    amax = t.abs().amax(dim=-1)
    s = torch.where(amax > 0, amax / torch.tensor(448.0, dtype=torch.float32), torch.ones_like(amax))
    codes = (t / s[..., None]).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    codes[codes == 0x80] = 0
    return codes, s.numpy()


def _bf16_sweep_rows(amax):
    """Every finite bf16 value v with |v| <= amax, 127 per row, each row led by the anchor amax (so
    that every row's scale is amax / 448)."""
    v = synth.bf16_bits_to_f32(np.arange(65536, dtype=np.uint32).astype(np.uint16))
    v = v[np.isfinite(v) & (np.abs(v) <= amax)]
    n = (v.size + 126) // 127
    rows = np.zeros((n, 128), dtype=np.float32)
    rows[:, 0] = amax
    body = rows[:, 1:].reshape(-1)
    body[: v.size] = v
    rows[:, 1:] = body.reshape(n, 127)
    return rows


@pytest.mark.parametrize("amax", [448.0, 1.0, 3.0, 0.1015625, 1232.0, 2.0 ** -10, 0.00506591796875,
                                  37.0, 3.3895313892515355e38])
def test_fp8_rows_fp32_decisions_bit_exact_exhaustive_bf16(amax):
    """fp8_quantize_rows(kernel_fp32=True) against the torch route, bit for bit, on every finite bf16
    value under each anchor (the anchors are bf16 values: scales 1, non-powers of two, tiny, huge)."""
    rows = _bf16_sweep_rows(np.float32(amax))
    codes, s, deq = O.fp8_quantize_rows(rows.astype(np.float64), kernel_fp32=True)
    ref_codes, ref_s = _torch_fp32_route(rows)
    np.testing.assert_array_equal(s, ref_s.astype(np.float64))
    np.testing.assert_array_equal(codes, ref_codes)
    np.testing.assert_array_equal(deq, O.e4m3_decode(ref_codes) * ref_s.astype(np.float64)[:, None])


def test_fp8_rows_fp32_decisions_gaussian_zero_and_ties():
    """Gaussian rows at several scales (bf16 values), all-zero rows, and exact E4M3FN ties: with the
    scale a power of two, v / s lands exactly on the midpoint of two neighbouring codes and must go to
    the even one."""
    r = np.random.default_rng(77)
    g = synth.bf16_bits_to_f32(synth.f32_to_bf16_bits(
        r.standard_normal((400, 128)).astype(np.float32) * np.repeat([1e-3, 0.02, 1.28, 40.0], 100)[:, None]))
    g[5] = 0.0
    c, s, _ = O.fp8_quantize_rows(g.astype(np.float64), kernel_fp32=True)
    rc, rs = _torch_fp32_route(g)
    np.testing.assert_array_equal(c, rc)
    np.testing.assert_array_equal(s, rs.astype(np.float64))
    assert s[5] == 1.0 and (c[5] == 0).all()
    tab = O.e4m3_table()
    mids = ((tab[1:] + tab[:-1]) / 2)[:125]                    # ties below 448
    for k in (0, 3, -7):
        row = np.concatenate([[448.0], mids, [0.0, -mids[40]]]) * 2.0 ** k   # scale exactly 2^k
        c, s, _ = O.fp8_quantize_rows(row[None], kernel_fp32=True)
        assert s[0] == 2.0 ** k
        lower = np.arange(125)
        np.testing.assert_array_equal(c[0, 1:126], np.where(lower % 2 == 0, lower, lower + 1))
        np.testing.assert_array_equal(c[0], _torch_fp32_route(row[None])[0][0])


# ------------------------------------------------------------------------------- indexer keys
def test_compress_ik_brute_force_own_logits_no_norm_no_rope():
    """Indexer keys: each block's tokens softmax-weighted by the indexer's own logits, then nothing
    else (no RMSNorm, no rotation), brute force on T <= 16; fp8 mode: the nearest E4M3FN code (ties to
    even) of key / (absmax / 448), found by searching all finite codes."""
    for (m, ov, T, dI) in ((4, 4, 15, 16), (4, 0, 16, 128), (3, 2, 14, 64)):
        r = np.random.default_rng(T + dI)
        ik, s = r.standard_normal((T, dI)) * 2.0, r.standard_normal(T)
        got = O.compress_ik(ik, s, m, ov, fp8=False)
        assert got.shape == (T // m, dI)
        for i in range(T // m):
            toks = [j for j in range(T) if i * m - ov <= j < (i + 1) * m]
            e = [math.exp(s[j] - max(s[u] for u in toks)) for j in toks]
            for d in range(dI):
                brute = sum(e[a] * ik[j, d] for a, j in enumerate(toks)) / sum(e)
                assert abs(got[i, d] - brute) < 1e-12
        # no norm: the keys scale with the tokens (RMSNorm would undo it); one dominant logit picks
        # that token's raw vector (a rotation or norm would change it)
        np.testing.assert_allclose(O.compress_ik(5 * ik, s, m, ov, fp8=False), 5 * got, rtol=1e-13, atol=1e-12)
        s1 = np.zeros(T)
        s1[m + 1] = 80.0
        np.testing.assert_allclose(O.compress_ik(ik, s1, m, ov, fp8=False)[1], ik[m + 1], atol=1e-20)
        codes, sc, deq = O.compress_ik(ik, s, m, ov, fp8=True)
        tab = np.array([O.e4m3_value(c) for c in range(127)])
        for i in range(T // m):
            assert sc[i] == np.abs(got[i]).max() / 448.0
            for d in range(dI):
                x = got[i, d] / sc[i]
                dist = np.abs(tab - abs(x))
                best = np.flatnonzero(dist == dist.min())
                want = best[0] if best.size == 1 else best[best % 2 == 0][0]
                if x < 0 and want != 0:
                    want |= 0x80
                assert codes[i, d] == want
        np.testing.assert_allclose(deq, O.e4m3_decode(codes) * sc[:, None], rtol=0, atol=0)


# ------------------------------------------------------------------------------- indexer + top-k
def test_index_scores_brute_force():
    H, d, n = 3, 5, 7
    q, w, k = randn(H, d), randn(H), randn(n, d)
    got = O.index_scores(q, w, k)
    for s in range(n):
        ref = 0.0
        for h in range(H):
            dot = sum(q[h, i] * k[s, i] for i in range(d))
            ref += w[h] * (dot if dot > 0 else 0.0)
        assert abs(got[s] - ref) < 1e-12


def test_index_single_head_orders_by_relu_dot():
    q, k = randn(1, 16), randn(40, 16)
    sc = O.index_scores(q, np.ones(1), k)
    np.testing.assert_allclose(sc, np.maximum(k @ q[0], 0))


def test_topk_against_stable_sort_with_ties():
    sc = np.array([3.0, 1.0, 3.0, 2.0, 3.0, -1.0, 2.0])
    ref = sorted(range(len(sc)), key=lambda s: (-sc[s], s))
    for k in range(1, 10):
        got = O.topk_select(sc, k)
        want = sorted(ref[:k]) + [-1] * max(0, k - len(sc))
        assert list(got) == want
    x = randn(1000)
    np.testing.assert_array_equal(O.topk_select(x, 50), np.sort(np.argsort(-x, kind="stable")[:50]))


def test_visibility_is_strictly_block_causal():
    for m in (1, 4, 128):
        for t in range(0, 3 * m + 2):
            vis = [i for i in range(4 * m) if (i + 1) * m <= t]
            assert O.n_visible(t, m) == len(vis)
            # the block containing t itself is never visible
            assert t // m not in vis


# ------------------------------------------------------------------------------- attention
def _torch_attn(q, K, scale=None):
    """Textbook softmax attention in float64 via torch (one query row per head)."""
    qt = torch.from_numpy(q)[None, :, None, :]           # [1, H, 1, D]
    kt = torch.from_numpy(K)[None, None].expand(1, q.shape[0], K.shape[0], K.shape[1])
    kw = {} if scale is None else {"scale": scale}
    return torch.nn.functional.scaled_dot_product_attention(qt, kt, kt, **kw)[0, :, 0].numpy()


def test_attend_sink_minus_inf_is_textbook_softmax():
    H, n, t = 4, 9, 77
    q, K = randn(H, 512), randn(n, 512)
    g = np.ones(512)
    got = O.attend_one(q, g, K, np.full(H, -np.inf), t, 1.0 / math.sqrt(512))
    qh = np.stack([O.rope(O.rmsnorm(q[h], g, 1e-6), t) for h in range(H)])
    ref = _torch_attn(qh, K)                               # default scale 1/sqrt(512)
    ref = np.stack([O.rope(ref[h], -t) for h in range(H)])
    np.testing.assert_allclose(got, ref, atol=1e-12)


def test_attend_sink_closed_form():
    H, n, t = 3, 11, 5
    q, K = randn(H, 512), randn(n, 512)
    g = np.ones(512)
    sc = 1.0 / math.sqrt(512)
    base = O.attend_one(q, g, K, np.full(H, -np.inf), t, sc)
    z = np.array([-2.0, 0.0, 3.0])
    got = O.attend_one(q, g, K, z, t, sc)
    for h in range(H):
        qh = O.rope(O.rmsnorm(q[h], g, 1e-6), t)
        S = np.exp(sc * (K @ qh)).sum()
        np.testing.assert_allclose(got[h], base[h] * S / (S + math.exp(z[h])), atol=1e-12)


def test_attend_single_key_returns_normed_token():
    x = randn(30, 512)
    q = randn(1, 2, 512)
    g = 0.5 + RNG.random(512)
    win = O.window_entries(x, g)
    for t in (0, 17, 29):
        o = O.hca_attend_one(q[0], np.ones(512), np.zeros((0, 512)), 128, win, [-np.inf] * 2, t, 1,
                             1.0 / math.sqrt(512))
        np.testing.assert_allclose(o[0], O.rmsnorm(x[t], g, 1e-6), atol=1e-12)
        np.testing.assert_allclose(o[1], O.rmsnorm(x[t], g, 1e-6), atol=1e-12)


def test_hca_m1_window1_equals_causal_mqa_and_torch():
    T, H = 13, 2
    kv, s = randn(T, 512), randn(T)
    q = randn(T, H, 512)
    sink = np.full(H, -np.inf)
    got = O.hca_layer(kv, s, q, sink, list(range(T)), m=1, W=1)
    ref = O.causal_mqa(q, np.ones(512), kv, np.ones(512), 1.0 / math.sqrt(512))
    np.testing.assert_allclose(got, ref, atol=1e-12)
    # the textbook reference itself against torch's causal attention in float64
    K = np.stack([O.rope(O.rmsnorm(kv[j], np.ones(512), 1e-6), j) for j in range(T)])
    for h in range(H):
        Q = np.stack([O.rope(O.rmsnorm(q[t, h], np.ones(512), 1e-6), t) for t in range(T)])
        o = torch.nn.functional.scaled_dot_product_attention(
            torch.from_numpy(Q)[None], torch.from_numpy(K)[None], torch.from_numpy(K)[None],
            is_causal=True)[0].numpy()
        o = np.stack([O.rope(o[t], -t) for t in range(T)])
        np.testing.assert_allclose(ref[:, h], o, atol=1e-12)


def _csa_inputs(T, H=4, HI=4, dI=16, seed=0):
    r = np.random.default_rng(seed)
    return dict(kv_tok=r.standard_normal((T, 512)), kv_score=r.standard_normal(T),
                ik_tok=r.standard_normal((T, dI)), ik_score=r.standard_normal(T),
                q=r.standard_normal((T, H, 512)), q_idx=r.standard_normal((T, HI, dI)),
                w_idx=r.standard_normal((T, HI)), sink=r.standard_normal(H))


def test_csa_topk_covering_all_equals_hca_m4():
    T = 40
    a = _csa_inputs(T)
    pos = [3, 8, 21, 39]
    o_csa, sel, _ = O.csa_layer(a["kv_tok"], a["kv_score"], a["ik_tok"], a["ik_score"], a["q"][pos],
                                a["q_idx"][pos], a["w_idx"][pos], a["sink"], pos, m=4, ov=4, W=6,
                                k=64, fp8=True)
    # same cache, dense over all visible entries: HCA attend with m = 4 on the CSA entries
    ent = O.compress_kv(a["kv_tok"], a["kv_score"], 4, 4, np.ones(512))
    win = O.window_entries(a["kv_tok"], np.ones(512))
    for i, t in enumerate(pos):
        ref = O.hca_attend_one(a["q"][t], np.ones(512), ent, 4, win, a["sink"], t, 6, 1 / math.sqrt(512))
        np.testing.assert_allclose(o_csa[i], ref, atol=1e-12)
        assert (sel[i] >= 0).sum() == t // 4


def test_csa_sparse_selection_changes_output():
    T = 64
    a = _csa_inputs(T, seed=3)
    pos = [63]
    o_k2, sel, sc = O.csa_layer(a["kv_tok"], a["kv_score"], a["ik_tok"], a["ik_score"], a["q"][pos],
                                a["q_idx"][pos], a["w_idx"][pos], a["sink"], pos, k=2, W=4)
    assert list(sel[0][:2]) == sorted(np.argsort(-sc[0], kind="stable")[:2])
    o_all, _, _ = O.csa_layer(a["kv_tok"], a["kv_score"], a["ik_tok"], a["ik_score"], a["q"][pos],
                              a["q_idx"][pos], a["w_idx"][pos], a["sink"], pos, k=64, W=4)
    assert np.abs(o_k2 - o_all).max() > 1e-3


@pytest.mark.parametrize("delta", [12345, (1 << 20) - 7])
def test_position_shift_invariance(delta):
    T = 36
    a = _csa_inputs(T, seed=5)
    pos = [7, 20, 35]
    kw = dict(m=4, ov=4, W=8, k=3, fp8=True)
    o0, s0, _ = O.csa_layer(a["kv_tok"], a["kv_score"], a["ik_tok"], a["ik_score"], a["q"][pos],
                            a["q_idx"][pos], a["w_idx"][pos], a["sink"], pos, rope_offset=0, **kw)
    o1, s1, _ = O.csa_layer(a["kv_tok"], a["kv_score"], a["ik_tok"], a["ik_score"], a["q"][pos],
                            a["q_idx"][pos], a["w_idx"][pos], a["sink"], pos, rope_offset=delta, **kw)
    np.testing.assert_array_equal(s0, s1)
    np.testing.assert_allclose(o0, o1, atol=1e-9)
    h0 = O.hca_layer(a["kv_tok"], a["kv_score"], a["q"][pos], a["sink"], pos, m=8, W=5)
    h1 = O.hca_layer(a["kv_tok"], a["kv_score"], a["q"][pos], a["sink"], pos, m=8, W=5, rope_offset=delta)
    np.testing.assert_allclose(h0, h1, atol=1e-9)


# ------------------------------------------------------------------------------- grouped projection
def test_grouped_out_proj_block_diagonal():
    M, H, c, g, dg, d = 3, 4, 512, 2, 6, 5
    o = randn(M, H * c)
    wg, wo = randn(g, dg, H * c // g), randn(d, g * dg)
    z, y = O.grouped_out_proj(o, wg, wo)
    bd = scipy.linalg.block_diag(*[wg[j] for j in range(g)])      # [g*dg, H*c]
    np.testing.assert_allclose(z, np.matmul(o, bd.T), atol=1e-10)
    np.testing.assert_allclose(y, np.matmul(np.matmul(o, bd.T), wo.T), atol=1e-10)
    o2 = o.copy()
    o2[:, :H * c // g] = 0                                          # zero group 0's heads
    z2, _ = O.grouped_out_proj(o2, wg, wo)
    assert np.all(z2[:, :dg] == 0) and np.allclose(z2[:, dg:], z[:, dg:])
    z1, y1 = O.grouped_out_proj(o, randn(1, dg, H * c)[:, :, :], wo[:, :dg])
    assert z1.shape == (M, dg)


def test_grouped_out_proj_g1_is_two_matmuls():
    o, wg, wo = randn(2, 1024), randn(1, 7, 1024), randn(3, 7)
    z, y = O.grouped_out_proj(o, wg, wo)
    np.testing.assert_allclose(y, np.matmul(np.matmul(o, wg[0].T), wo.T), atol=1e-10)


# ------------------------------------------------------------------------------- mHC (Sinkhorn-Knopp)
def test_sigmoid_anchors():
    assert O.sigmoid(0.0) == 0.5
    assert abs(O.sigmoid(math.log(3.0)) - 0.75) < 1e-15          # 1 / (1 + 1/3)
    assert abs(O.sigmoid(-math.log(3.0)) - 0.25) < 1e-15


def test_sinkhorn_uniform_and_rank_one_closed_forms():
    n = 4
    assert np.allclose(O.sinkhorn(np.zeros((n, n))), 1.0 / n, atol=1e-15)
    # exp(a_i + b_j) is rank one: one round (rows, then columns) already gives the uniform matrix
    a, b = randn(n), randn(n)
    for it in (1, 20):
        assert np.allclose(O.sinkhorn(a[:, None] + b[None, :], it), 1.0 / n, atol=1e-14)


def test_sinkhorn_one_round_by_hand():
    """[[1,2],[3,4]]: rows -> [[1/3,2/3],[3/7,4/7]]; column sums 16/21, 26/21 -> [[7/16,7/13],[9/16,6/13]].
    Columns first would give [[3/7,4/7],[9/17,8/17]]: the order of the two normalisations is pinned."""
    got = O.sinkhorn(np.log(np.array([[1.0, 2.0], [3.0, 4.0]])), 1)
    want = np.array([[7 / 16, 7 / 13], [9 / 16, 6 / 13]])
    assert np.allclose(got, want, atol=1e-15, rtol=0)


def test_sinkhorn_2x2_limit_is_the_cross_ratio_form():
    """The doubly stochastic scaling of a positive [[a,b],[c,d]] is [[p,1-p],[1-p,p]] with
    p / (1-p) = sqrt(ad / bc) (the cross ratio ad/bc is invariant under row and column scaling)."""
    for a, b, c, d in [(1, 2, 3, 4), (5.0, 0.1, 0.3, 2.0), (1, 1, 1, 7)]:
        p = math.sqrt(a * d) / (math.sqrt(a * d) + math.sqrt(b * c))
        got = O.sinkhorn(np.log(np.array([[a, b], [c, d]], dtype=np.float64)), 500)
        assert np.allclose(got, [[p, 1 - p], [1 - p, p]], atol=1e-12)


def test_sinkhorn_rounds_are_row_shift_invariant_and_converge():
    L = randn(60, 4, 4, std=1.5)
    shift = randn(60, 4)
    for i in range(60):
        B = O.sinkhorn(L[i])
        assert np.allclose(B.sum(axis=0), 1.0, atol=1e-14)                 # columns: exact after each round
        assert np.abs(B.sum(axis=1) - 1.0).max() < 5e-2                   # rows: close after 20 rounds
        # the rows' L1 distance to 1 never grows from one round to the next, and vanishes in the limit
        errs = [np.abs(O.sinkhorn(L[i], k).sum(axis=1) - 1.0).sum() for k in range(1, 30)]
        assert all(e1 <= e0 + 1e-15 for e0, e1 in zip(errs, errs[1:]))
        assert np.abs(O.sinkhorn(L[i], 400).sum(axis=1) - 1.0).max() < 1e-9
        # a row shift of the logits is a row scaling, removed by the first row normalisation
        assert np.allclose(O.sinkhorn(L[i] + shift[i][:, None], 3), O.sinkhorn(L[i], 3), atol=1e-14)
        # a column shift is removed only in the limit
        assert np.allclose(O.sinkhorn(L[i] + shift[i][None, :], 400), O.sinkhorn(L[i], 400), atol=1e-10)


def test_mhc_mix_by_hand_and_stream_sum():
    """n = 2, one round: B = [[7/16,7/13],[9/16,6/13]] (above), C = sigmoid(log 3) = 3/4,
    A = sigmoid(0) = 1/2; every output written out by hand."""
    X = np.array([[[1.0, -2.0, 0.5], [4.0, 0.25, -1.0]]])
    y = np.array([[2.0, 1.0, -4.0]])
    L = np.concatenate([np.log([1.0, 2.0, 3.0, 4.0]), [math.log(3.0)] * 2, [0.0, 0.0]])[None, :]
    Xo, h = O.mhc_mix(X, y, L, iters=1)
    x0 = 7 / 16 * X[0, 0] + 7 / 13 * X[0, 1] + 0.75 * y[0]
    x1 = 9 / 16 * X[0, 0] + 6 / 13 * X[0, 1] + 0.75 * y[0]
    assert np.allclose(Xo[0], [x0, x1], atol=1e-14)
    assert np.allclose(h[0], 0.5 * (x0 + x1), atol=1e-14)
    # with y = 0 the streams' sum is kept whatever the rows sum to (columns sum to 1): B X, not B^T X
    Xr = randn(6, 4, 8)
    Lr = randn(6, 24, std=2.0)
    Xo, _ = O.mhc_mix(Xr, np.zeros((6, 8)), Lr, iters=1)
    assert np.allclose(Xo.sum(axis=1), Xr.sum(axis=1), atol=1e-12)


# ------------------------------------------------------------------------------- input projections
def test_input_projection_brute_force_and_split():
    h = randn(3, 7)
    w = randn(11, 7)                       # 2 + 1 + 5 columns used, 3 padding rows
    parts = O.input_projection(h, w, [2, 1, 5])
    assert [p.shape for p in parts] == [(3, 2), (3, 1), (3, 5)]
    brute = [[sum(h[m, k] * w[n, k] for k in range(7)) for n in range(8)] for m in range(3)]
    assert np.allclose(np.concatenate(parts, axis=1), brute, atol=1e-12)


def test_residual_chain_closed_forms():
    h = randn(2, 5)
    assert np.array_equal(O.residual(h, np.zeros_like(h)), h)
    assert np.array_equal(O.residual(h, -h), np.zeros_like(h))
