"""GPU parity of the input projections (one pass over concatenated weights, outputs scattered into
bf16 / fp32 segments), the grouped projection with the residual added, and a chained 4-layer decode
step (projections -> token append -> index/top-k -> attention -> projection + residual) checked layer by
layer against the oracle on the GPU's own intermediate hidden states."""
import math

import numpy as np
import pytest
import torch

import long_context_sparse_17_amd as L
import oracle as O
import synth
from lcs_testutil import assert_close, check_topk_row, from_bits, index_oracle_row, to_np_bf16

pytestmark = pytest.mark.gpu
DEV = "cuda"


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64) if t.dtype == torch.float32 else to_np_bf16(t)


@pytest.mark.parametrize("M,d", [(1, 4096), (8, 4096), (5, 8192)])
def test_input_proj_segments(M, d):
    h = synth.normal_bf16((M, d), 1.0, 180 + M, 1)
    widths = [100, 1, 33, 300, 16]
    n_rows = (sum(widths) + 15) // 16 * 16 + 16              # plus a padding block
    w = synth.normal_bf16((n_rows, d), 0.02, 180 + M, 2)
    dst = [torch.full((M, 128), 7.0, dtype=torch.bfloat16, device=DEV),     # ld 128 > width 100
           torch.full((M,), 7.0, dtype=torch.float32, device=DEV),          # one column, 1-D
           torch.full((M, 40), 7.0, dtype=torch.float32, device=DEV),
           torch.full((M, 300), 7.0, dtype=torch.bfloat16, device=DEV),
           torch.full((M, 16), 7.0, dtype=torch.float32, device=DEV)]
    L.input_proj(from_bits(h), from_bits(w), list(zip(widths, dst)))
    torch.cuda.synchronize()
    ref = O.input_projection(synth.bf16_bits_to_f64(h), synth.bf16_bits_to_f64(w), widths)
    for i, (wd, t) in enumerate(zip(widths, dst)):
        got = f64(t).reshape(M, -1)
        assert_close(got[:, :wd], ref[i], f"segment {i}")
        assert np.all(got[:, wd:] == 7.0), "columns past a segment's width must not be written"


@pytest.mark.parametrize("M,H,g,d_g,d,inplace", [(8, 64, 8, 1024, 4096, False), (8, 64, 8, 1024, 4096, True),
                                                  (37, 8, 2, 64, 96, False), (200, 16, 2, 128, 256, True),
                                                  (200, 16, 2, 128, 256, False), (600, 16, 2, 256, 512, True),
                                                  (600, 16, 2, 256, 512, False)])
def test_grouped_out_proj_residual(M, H, g, d_g, d, inplace):
    o = synth.normal_bf16((M, H * 512), 1.0, 190 + M, 1)
    wg = synth.normal_bf16((g, d_g, H // g * 512), 0.02, 190 + M, 2)
    wo = synth.normal_bf16((d, g * d_g), 0.02, 190 + M, 3)
    r = synth.normal_bf16((M, d), 1.0, 190 + M, 4)
    r_dev = from_bits(r)
    y = r_dev if inplace else torch.empty((M, d), dtype=torch.bfloat16, device=DEV)
    L.grouped_out_proj_residual(from_bits(o), from_bits(wg), from_bits(wo), r_dev, H=H, y=y)
    torch.cuda.synchronize()
    _, yref = O.grouped_out_proj(synth.bf16_bits_to_f64(o), synth.bf16_bits_to_f64(wg), synth.bf16_bits_to_f64(wo))
    assert_close(to_np_bf16(y), O.residual(synth.bf16_bits_to_f64(r), yref), f"residual M={M} inplace={inplace}")


def test_chained_decode_step_layer_by_layer():
    from long_context_sparse_17_amd.pipeline import RING, ChainedStack, CsaDecodeLayer, hybrid_stack
    B, ctx = 2, 8192
    layers = hybrid_stack(B=B, ctx=ctx, k=1024, device=DEV)
    stack = ChainedStack(layers)
    stack.h.copy_(stack.h0)
    ones = np.ones(512)
    scale = 1.0 / math.sqrt(512)
    bits = lambda x: x.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16)  # noqa: E731
    for Lr, w, segs in zip(layers, stack.w_in, stack.segs):
        h_in = to_np_bf16(stack.h)
        L.input_proj(stack.h, w, segs)
        Lr.step()
        torch.cuda.synchronize()
        # (a) the projections, from the GPU's hidden state
        ref = O.input_projection(h_in, to_np_bf16(w), [wd for wd, _ in segs])
        for i, (wd, t) in enumerate(segs):
            assert_close(f64(t).reshape(B, -1)[:, :wd], ref[i], f"projection segment {i}")
        # (b) attention on the layer's caches, ring and projected inputs
        t = Lr.t
        o_all = []
        for b in range(B):
            new_win = O.rope(O.rmsnorm(synth.bf16_bits_to_f64(bits(Lr.new_tok[b, 0])), ones, 1e-6), t)
            if isinstance(Lr, CsaDecodeLayer):
                kdeq = O.e4m3_decode(Lr.ik_cache[b].cpu().numpy()) * Lr.ik_scale[b].cpu().numpy()[:, None].astype(np.float64)
                sc, bound = index_oracle_row(bits(Lr.q_idx[b, 0]), bits(Lr.w_idx[b, 0]), kdeq[: t // Lr.m], True)
                gsel = Lr.topk[b, 0].cpu().numpy()
                check_topk_row(gsel, sc, Lr.k, bound)
                keys = [to_np_bf16(Lr.kv_cache[b])[gsel[gsel >= 0]]]
            else:
                keys = [to_np_bf16(Lr.kv_cache[b])[: t // Lr.m]]
            ring = to_np_bf16(Lr.ring[b])
            keys = np.concatenate(keys + [ring[[j % RING for j in range(t - 127, t)]], new_win[None]])
            o = O.attend_one(to_np_bf16(Lr.q[b, 0]), ones, keys, Lr.sink.cpu().numpy().astype(np.float64), t, scale)
            assert_close(to_np_bf16(Lr.o[b, 0]), o, f"layer o b={b}")
            o_all.append(to_np_bf16(Lr.o[b, 0]).reshape(-1))
        # (c) h <- h + projection of the GPU's o
        _, y = O.grouped_out_proj(np.stack(o_all), to_np_bf16(Lr.w_g), to_np_bf16(Lr.w_o))
        assert_close(to_np_bf16(stack.h), O.residual(h_in, y), "residual chain")
