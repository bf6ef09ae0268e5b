"""The allocation-free grouped projection (z in the library's static device scratch) against the
workspace entry point, through the C ABI: bit-identical outputs on two calls in a row, the second with
fewer rows, and the scratch limit checked on the host."""
import ctypes

import numpy as np
import pytest
import torch

import long_context_sparse_17_amd as L
import synth
from lcs_testutil import from_bits

pytestmark = pytest.mark.gpu
DEV = "cuda"


def _inputs(M, H, g, d_g, d, cfg):
    o = from_bits(synth.normal_bf16((M, H * 512), 0.3, cfg, 1))
    wg = from_bits(synth.normal_bf16((g, d_g, H * 512 // g), 0.02, cfg, 2))
    wo = from_bits(synth.normal_bf16((d, g * d_g), 0.02, cfg, 3))
    return o, wg, wo


@pytest.mark.parametrize("shapes", [[(8, 64, 8, 1024, 4096), (3, 64, 8, 1024, 4096)],
                                    [(37, 16, 2, 64, 96), (5, 16, 2, 64, 96)]])
def test_noalloc_matches_workspace_entry_point(shapes):
    for i, (M, H, g, d_g, d) in enumerate(shapes):
        print(f"noalloc call {i}: M={M} H={H} g={g} d_g={d_g} d={d}", flush=True)
        o, wg, wo = _inputs(M, H, g, d_g, d, 90 + i)
        y_ref = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
        y = torch.full((M, d), float("nan"), dtype=torch.bfloat16, device=DEV)
        L.grouped_out_proj(o, wg, wo, H=H, y=y_ref)
        L.grouped_out_proj_noalloc(o, wg, wo, H=H, y=y)
        torch.cuda.synchronize()
        assert torch.equal(y.view(torch.int16), y_ref.view(torch.int16)), f"call {i} differs"


def test_noalloc_rejects_oversized_shape_and_allocates_nothing():
    M, H, g, d_g, d = 8, 64, 8, 1024, 4096
    o, wg, wo = _inputs(M, H, g, d_g, d, 95)
    y = torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    torch.cuda.synchronize()
    before = torch.cuda.memory_allocated()
    L.grouped_out_proj_noalloc(o, wg, wo, H=H, y=y)
    torch.cuda.synchronize()
    assert torch.cuda.memory_allocated() == before
    big = L.lib().grouped_out_proj_noalloc_max_bytes() // (g * d_g * 2) + 1
    st = L.lib().grouped_out_proj_noalloc(ctypes.c_void_p(o.data_ptr()), ctypes.c_void_p(wg.data_ptr()),
                                          ctypes.c_void_p(wo.data_ptr()), big, H, 512, g, d_g, d,
                                          ctypes.c_void_p(y.data_ptr()), None)
    assert st == L.LCS_ERR_SCRATCH
