"""C-ABI contract tests (no GPU): the library loads, exports every symbol include/lcs.h declares, and
rejects bad arguments on the host before anything is launched."""
import ctypes
import os
import re

import pytest

import long_context_sparse_17_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lcs.h")


def declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(", src, flags=re.M)
    return sorted(set(names))


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(L.LIB_PATH):
        pytest.fail("liblcs.so is not built (run __graft_entry__.build())")
    return L.lib()


def test_every_declared_symbol_is_exported_and_bound(lib):
    names = declared_functions()
    assert len(names) >= 13
    for n in names:
        assert hasattr(lib, n), n
        assert n in L.SIGNATURES, f"binding misses {n}"
    assert set(L.SIGNATURES) == set(names)


def test_version_and_status_strings(lib):
    assert lib.lcs_version() >= 10000
    for code, txt in [(0, b"ok"), (1, b"invalid argument"), (3, b"workspace too small")]:
        assert lib.lcs_status_string(code) == txt


def test_workspace_queries_are_positive_and_monotone(lib):
    a = lib.csa_index_topk_workspace(8, 1, 262144, 1024)
    b = lib.csa_index_topk_workspace(8, 1, 262145, 1024)
    assert 0 < a <= b
    assert lib.csa_index_topk_workspace(0, 1, 10, 1) == 0
    assert lib.lcs_attend_workspace(8, 1, 64, 8192 + 128) > 8 * 64 * 512 * 4
    assert lib.grouped_out_proj_workspace(8, 8, 1024) >= 8 * 8 * 1024 * 2


FAKE = ctypes.c_void_p(1 << 20)   # aligned, never dereferenced: validation fails first


def test_attend_rejects_bad_arguments(lib):
    args = [FAKE, FAKE, FAKE, 100, FAKE, 16, FAKE, 200, 0, 128, FAKE, FAKE, 0, 1, 1, 64, 512, 0.04, 1e-6, 1e4,
            FAKE, FAKE, 1 << 30, None]
    bad_c = list(args); bad_c[16] = 256
    assert lib.csa_attend(*bad_c) == L.LCS_ERR_UNSUPPORTED
    bad_h = list(args); bad_h[15] = 65
    assert lib.csa_attend(*bad_h) == L.LCS_ERR_UNSUPPORTED
    null_q = list(args); null_q[0] = None
    assert lib.csa_attend(*null_q) == L.LCS_ERR_ARG
    small_ws = list(args); small_ws[22] = 0
    assert lib.csa_attend(*small_ws) == L.LCS_ERR_WORKSPACE
    mis = list(args); mis[0] = ctypes.c_void_p((1 << 20) + 2)
    assert lib.csa_attend(*mis) == L.LCS_ERR_ARG
    big_k = list(args); big_k[5] = 4096
    assert lib.csa_attend(*big_k) == L.LCS_ERR_UNSUPPORTED
    neg_scale = list(args); neg_scale[17] = -1.0
    assert lib.csa_attend(*neg_scale) == L.LCS_ERR_ARG


def test_index_rejects_bad_arguments(lib):
    base = [FAKE, FAKE, FAKE, FAKE, 1000, L.LCS_IK_FP8, FAKE, 1000, 2, 1, 64, 128, 4, 64, FAKE, None, FAKE,
            1 << 30, None]
    assert lib.csa_index_topk(*[a if i != 11 else 64 for i, a in enumerate(base)]) == L.LCS_ERR_UNSUPPORTED
    assert lib.csa_index_topk(*[a if i != 10 else 65 for i, a in enumerate(base)]) == L.LCS_ERR_UNSUPPORTED
    assert lib.csa_index_topk(*[a if i != 13 else 4096 for i, a in enumerate(base)]) == L.LCS_ERR_UNSUPPORTED
    assert lib.csa_index_topk(*[a if i != 17 else 16 for i, a in enumerate(base)]) == L.LCS_ERR_WORKSPACE
    assert lib.csa_index_topk(*[a if i != 4 else 999 for i, a in enumerate(base)]) == L.LCS_ERR_ARG
    assert lib.csa_index_topk(*[a if i != 5 else 7 for i, a in enumerate(base)]) == L.LCS_ERR_UNSUPPORTED
    assert lib.csa_index_topk(*[a if i != 3 else None for i, a in enumerate(base)]) == L.LCS_ERR_ARG
    # many rows of one query each: the row-per-workgroup grids would pass 65535 rows in y
    assert lib.csa_index_topk(*[a if i != 8 else 70000 for i, a in enumerate(base)]) == L.LCS_ERR_UNSUPPORTED
    bf16 = [a if i not in (3, 5) else (None if i == 3 else L.LCS_IK_BF16) for i, a in enumerate(base)]
    assert lib.csa_index_topk(*[a if i != 8 else 70000 for i, a in enumerate(bf16)]) == L.LCS_ERR_UNSUPPORTED


def test_compress_rejects_tokens_outside_the_given_columns(lib):
    # blocks 10..11 of m=4, ov=4 need tokens 36..47; columns start at tok0 = 40
    args = [FAKE, FAKE, None, None, 1, 8, 40, 10, 2, 4, 4, 512, 0, FAKE, 1e-6, 1e4, 0, FAKE, 100, 0, None, None, 0,
            0, None]
    assert lib.csa_compress_kv(*args) == L.LCS_ERR_ARG
    ok_cols = list(args); ok_cols[6] = 36; ok_cols[5] = 12
    bad_c = list(ok_cols); bad_c[11] = 128
    assert lib.csa_compress_kv(*bad_c) == L.LCS_ERR_UNSUPPORTED
    bad_ld = list(ok_cols); bad_ld[18] = 11
    assert lib.csa_compress_kv(*bad_ld) == L.LCS_ERR_ARG
    bad_ov = list(ok_cols); bad_ov[10] = 17
    assert lib.csa_compress_kv(*bad_ov) == L.LCS_ERR_UNSUPPORTED
    # HCA path: overlap is always 0; m = 128 blocks need 128 columns each
    assert lib.hca_compress_kv(FAKE, FAKE, 1, 100, 0, 0, 1, 128, 512, FAKE, 1e-6, 1e4, 0, FAKE, 10, 0, None) == \
        L.LCS_ERR_ARG


def test_decode_append_rejects_bad_arguments(lib):
    need = lib.kv_decode_state_bytes(8)
    assert need == 8 * 2 * (512 + 128 + 8) * 4
    # kv_tok, kv_score, ik_tok, ik_score, pos, B, m, ov, c, dI, gamma, eps, theta, offset, state, state_bytes,
    # kv_dtype, win, win_scale, win_ld, ring_cap, kv_out, kv_scale, kv_ld, kv_ring, ik_out, ik_scale, ik_ld,
    # ik_dtype, stream
    good = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 4, 512, 128, FAKE, 1e-6, 1e4, 0, FAKE, need, L.LCS_KV_BF16, FAKE, None,
            256, 256, FAKE, None, 1000, 0, FAKE, FAKE, 1000, L.LCS_IK_FP8, None]
    def call(**kw):
        a = list(good)
        for i, v in kw.items():
            a[int(i[1:])] = v
        return lib.kv_decode_append(*a)
    assert call(a15=need - 1) == L.LCS_ERR_WORKSPACE
    assert call(a7=5) == L.LCS_ERR_UNSUPPORTED            # overlap > m: a token in three blocks
    assert call(a8=256) == L.LCS_ERR_UNSUPPORTED           # c != 512
    assert call(a9=96) == L.LCS_ERR_UNSUPPORTED            # dI
    assert call(a4=None) == L.LCS_ERR_ARG                  # positions
    assert call(a19=100) == L.LCS_ERR_ARG                  # win_ld < ring_cap
    assert call(a24=1001) == L.LCS_ERR_ARG                 # kv_ring > kv_ld
    assert call(a26=None) == L.LCS_ERR_ARG                 # fp8 keys need scales
    assert call(a28=7) == L.LCS_ERR_UNSUPPORTED            # key dtype
    assert call(a16=5) == L.LCS_ERR_UNSUPPORTED            # K=V dtype
    assert call(a16=L.LCS_KV_FP8) == L.LCS_ERR_ARG         # fp8 K=V rows need their scales
    assert call(a16=L.LCS_KV_FP8, a22=FAKE) == L.LCS_ERR_ARG   # ... the ring's too
    assert call(a6=0) == L.LCS_ERR_ARG


def test_index_topk_append_checks_both_argument_sets(lib):
    """The fused selection + append call applies each entry point's checks, all on the host."""
    ws_need = lib.csa_index_topk_workspace(8, 1, 1000, 64)
    need = lib.kv_decode_state_bytes(8)
    index = [FAKE, FAKE, FAKE, FAKE, 1000, L.LCS_IK_FP8, FAKE, 1000, 8, 1, 64, 128, 4, 64, FAKE, None, FAKE, ws_need]
    append = [FAKE, FAKE, FAKE, FAKE, FAKE, 8, 4, 4, 512, 128, FAKE, 1e-6, 1e4, 0, FAKE, need, L.LCS_KV_BF16, FAKE,
              None, 256, 256, FAKE, None, 1000, 0, FAKE, FAKE, 1000, L.LCS_IK_FP8]
    def call(i=None, a=None):
        ix, ap = list(index), list(append)
        for k, v in (i or {}).items():
            ix[k] = v
        for k, v in (a or {}).items():
            ap[k] = v
        return lib.csa_index_topk_append(*ix, *ap, None)
    assert call(i={17: 16}) == L.LCS_ERR_WORKSPACE          # selection workspace too small
    assert call(i={13: 4096}) == L.LCS_ERR_UNSUPPORTED      # k
    assert call(a={15: need - 1}) == L.LCS_ERR_WORKSPACE    # decode state too small
    assert call(a={7: 5}) == L.LCS_ERR_UNSUPPORTED          # overlap > m
    assert call(a={4: None}) == L.LCS_ERR_ARG               # append positions
    assert call(a={26: None}) == L.LCS_ERR_ARG              # fp8 keys of the append need scales


def test_kv8_entry_points_reject_bad_arguments(lib):
    assert lib.kv_quantize_fp8(FAKE, 0, FAKE, FAKE, None) == L.LCS_ERR_ARG
    assert lib.kv_quantize_fp8(ctypes.c_void_p((1 << 20) + 8), 4, FAKE, FAKE, None) == L.LCS_ERR_ARG   # alignment
    # csa_attend_kv8 without row scales
    args = [FAKE, FAKE, FAKE, None, 100, FAKE, 16, FAKE, FAKE, 256, 256, 128, FAKE, FAKE, 0, 1, 1, 64, 512, 0.04,
            1e-6, 1e4, FAKE, FAKE, 1 << 30, None]
    assert lib.csa_attend_kv8(*args) == L.LCS_ERR_ARG
    hargs = [FAKE, FAKE, FAKE, FAKE, 100, 100, 4, FAKE, None, 256, 256, 128, FAKE, FAKE, 0, 1, 1, 64, 512, 0.04,
             1e-6, 1e4, FAKE, FAKE, 1 << 30, None]
    assert lib.hca_attend_kv8(*hargs) == L.LCS_ERR_ARG  # window keys without their scales


def test_kv8_attend_without_window_passes_validation(lib):
    """window = 0 with no ring (codes and scales NULL) is a valid call on both fp8 entry points: the
    checks get as far as the workspace (too small here, so nothing launches)."""
    args = [FAKE, FAKE, FAKE, FAKE, 100, FAKE, 300, None, None, 0, 0, 0, FAKE, FAKE, 0, 1, 1, 64, 512, 0.04,
            1e-6, 1e4, FAKE, FAKE, 16, None]
    assert lib.csa_attend_kv8(*args) == L.LCS_ERR_WORKSPACE
    hargs = [FAKE, FAKE, FAKE, FAKE, 100, 100, 4, None, None, 0, 0, 0, FAKE, FAKE, 0, 1, 1, 64, 512, 0.04,
             1e-6, 1e4, FAKE, FAKE, 16, None]
    assert lib.hca_attend_kv8(*hargs) == L.LCS_ERR_WORKSPACE
    # a window with no ring stays an argument error
    bad = list(hargs); bad[11] = 128
    assert lib.hca_attend_kv8(*bad) == L.LCS_ERR_ARG


def test_projection_and_mhc_entry_points_reject_bad_arguments(lib):
    widths = (ctypes.c_int * 2)(100, 1)
    dsts = (ctypes.c_void_p * 2)(1 << 20, 1 << 21)
    lds = (ctypes.c_int64 * 2)(128, 1)
    f32 = (ctypes.c_int * 2)(0, 1)
    args = [FAKE, 8, 4096, FAKE, 112, 2, widths, dsts, lds, f32, None]
    bad_m = list(args); bad_m[1] = 9
    assert lib.input_proj(*bad_m) == L.LCS_ERR_UNSUPPORTED       # decode rows only
    bad_d = list(args); bad_d[2] = 1000
    assert lib.input_proj(*bad_d) == L.LCS_ERR_UNSUPPORTED
    bad_rows = list(args); bad_rows[4] = 100
    assert lib.input_proj(*bad_rows) == L.LCS_ERR_UNSUPPORTED    # weight rows not a multiple of 16
    short = list(args); short[4] = 96
    assert lib.input_proj(*short) == L.LCS_ERR_ARG               # segments wider than the weights
    narrow = (ctypes.c_int64 * 2)(64, 1)
    bad_ld = list(args); bad_ld[8] = narrow
    assert lib.input_proj(*bad_ld) == L.LCS_ERR_ARG              # row stride below the width
    assert lib.grouped_out_proj_residual(FAKE, FAKE, FAKE, None, 8, 64, 512, 8, 1024, 4096, FAKE, FAKE, 1 << 30,
                                         None) == L.LCS_ERR_ARG
    assert lib.mhc_sinkhorn(FAKE, 10, 9, 20, FAKE, None) == L.LCS_ERR_UNSUPPORTED      # n > 8
    assert lib.mhc_sinkhorn(FAKE, 10, 4, 0, FAKE, None) == L.LCS_ERR_ARG               # no rounds
    assert lib.mhc_mix(FAKE, FAKE, FAKE, 4, 4, 100, 20, FAKE, None, None) == L.LCS_ERR_UNSUPPORTED  # d % 8


def test_out_proj_rejects_bad_grouping(lib):
    assert lib.grouped_out_proj(FAKE, FAKE, FAKE, 8, 64, 512, 7, 1024, 4096, FAKE, FAKE, 1 << 30, None) == \
        L.LCS_ERR_UNSUPPORTED
    assert lib.grouped_out_proj(FAKE, FAKE, FAKE, 8, 64, 512, 8, 1000, 4096, FAKE, FAKE, 1 << 30, None) == \
        L.LCS_ERR_UNSUPPORTED
    assert lib.grouped_out_proj(FAKE, FAKE, FAKE, 8, 64, 512, 8, 1024, 4096, FAKE, FAKE, 16, None) == \
        L.LCS_ERR_WORKSPACE


def test_out_proj_noalloc_limits_checked_on_the_host(lib):
    """The allocation-free projection rejects shapes whose z does not fit its static scratch, and bad
    shapes, before any HIP call (so on a machine without a GPU these return their codes)."""
    cap = lib.grouped_out_proj_noalloc_max_bytes()
    assert cap == 4 << 20
    assert lib.grouped_out_proj_noalloc(FAKE, FAKE, FAKE, 257, 64, 512, 8, 1024, 4096, FAKE, None) == \
        L.LCS_ERR_SCRATCH                                              # 257 * 8192 * 2 > 4 MiB
    assert lib.grouped_out_proj_noalloc(FAKE, FAKE, FAKE, 8, 64, 512, 7, 1024, 4096, FAKE, None) == \
        L.LCS_ERR_UNSUPPORTED
    assert lib.grouped_out_proj_noalloc(None, FAKE, FAKE, 8, 64, 512, 8, 1024, 4096, FAKE, None) == L.LCS_ERR_ARG
    assert lib.lcs_status_string(L.LCS_ERR_SCRATCH).startswith(b"shape needs more")


def test_timing_facility_without_launches(lib):
    assert lib.lcs_timing_enable(1) == 0
    ms = ctypes.c_double(-1)
    n = ctypes.c_int64(-1)
    assert lib.lcs_timing_read(b"attend", ctypes.byref(ms), ctypes.byref(n)) == 0
    assert n.value == 0 and ms.value == 0.0
    assert lib.lcs_timing_enable(0) == 0


def test_product_path_has_no_fallback():
    """The binding loads only liblcs.so; nothing in the package imports the oracle."""
    pkg = os.path.dirname(L.__file__)
    for root, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                txt = open(os.path.join(root, f), encoding="utf-8").read()
                assert "import oracle" not in txt and "from oracle" not in txt, f
