"""Decode-step drivers for one CSA or HCA layer, composed from the C-ABI entry points only.

A layer holds its device state (compressed caches, window ring, pooling state, weights,
workspaces) and `step()` enqueues one decode step for the query at token t = ctx of every
sequence, in the order the method runs it (page 1, "hybrid attention", CSA steps 1-4 / HCA):

  CSA: append token t (window-ring row; pooled state of the blocks containing t)
       -> indexer scores + top-k -> attention over the selected entries + window + sink
       -> grouped output projection
  HCA: append token t -> dense attention -> grouped output projection

The caches of tokens [0, ctx) come from the bulk compression; the pooled state of the block that is
still open at t (CSA: tokens ctx-4 .. ctx-1 of its overlap) is primed by appending those tokens to
empty slots (the block they end was compressed in bulk and is left alone).
No block ends at t = ctx, so the step finishes no entry; a block's entry is finished by the append
of its last token, once every m (CSA) or 128 (HCA) steps.
"""
from __future__ import annotations

import math

import torch

from . import (csa_attend, csa_compress_kv, csa_index_topk_append, csa_index_topk_workspace,
               attend_workspace,
               grouped_out_proj, grouped_out_proj_residual, grouped_out_proj_workspace, hca_attend_append,
               hca_compress_kv,
               input_proj, kv_decode_append, kv_decode_state_bytes, kv_quantize_fp8, workspace)

RING = 256          # window ring rows (>= the 128-token window)


class _Common:
    def __init__(self, B, ctx, H, W, g, d_g, d, device, weights_std, seed, kv8=False):
        self.B, self.ctx, self.H, self.W = B, ctx, H, W
        self.kv8 = kv8              # fp8 K=V storage (E4M3FN codes + one scale per row) for cache and ring
        self.g, self.d_g, self.d = g, d_g, d
        self.dev = device
        self.t = ctx
        gen = torch.Generator(device=device)
        gen.manual_seed(seed)

        def nrm(shape, std):
            x = torch.empty(shape, dtype=torch.float32, device=device)
            x.normal_(0.0, std, generator=gen)
            return x

        self._nrm = nrm
        self.gamma = torch.ones(512, dtype=torch.bfloat16, device=device)
        self.ring = torch.zeros((B, RING, 512), dtype=torch.uint8 if kv8 else torch.bfloat16, device=device)
        self.ring_sc = torch.zeros((B, RING), dtype=torch.float32, device=device) if kv8 else None
        self._ring_bf16 = None      # fp8 K=V: the bulk window fill writes bf16 here, then it is quantised
        self.stack_h = None         # in a chained stack: the hidden state [B, d] (input, and output in place)
        self.q_pos = torch.full((B, 1), ctx, dtype=torch.int64, device=device)
        self.state = torch.zeros(kv_decode_state_bytes(B), dtype=torch.uint8, device=device)  # empty slots
        self.sink = nrm((H,), 1.0)
        self.o = torch.empty((B, 1, H, 512), dtype=torch.bfloat16, device=device)
        self.y = torch.empty((B, d), dtype=torch.bfloat16, device=device)
        self.w_g = nrm((g, d_g, H * 512 // g), weights_std).to(torch.bfloat16)
        self.w_o = nrm((d, g * d_g), weights_std).to(torch.bfloat16)
        self.ws_proj = workspace(grouped_out_proj_workspace(B, g, d_g), device)
        self.new_tok = nrm((B, 1, 512), 1.28).to(torch.bfloat16)
        self.new_score = nrm((B, 1), 1.28)
        self.q = nrm((B, 1, H, 512), 1.28).to(torch.bfloat16)

    def fill_ring(self, tok, score, t0):
        """Window tokens [t0, t0 + T) of raw per-token vectors into the ring (m = 1 compression)."""
        T = tok.shape[1]
        ring = self.ring
        if self.kv8:
            self._ring_bf16 = torch.zeros((self.B, RING, 512), dtype=torch.bfloat16, device=self.dev)
            ring = self._ring_bf16
        hca_compress_kv(tok, score, tok0=t0, blk_begin=t0, n_blk=T, m=1, gamma_kv=self.gamma, kv_out=ring,
                        ring_cap=RING)

    def prime(self, tok, score, ik=None, iks=None, t0=0):
        """Append raw tokens [t0, t0 + T) one position at a time (kv_decode_append), so that the pooled
        state holds the open blocks' tokens."""
        for j in range(tok.shape[1]):
            pos = torch.full((self.B,), t0 + j, dtype=torch.int64, device=self.dev)
            kv_decode_append(tok[:, j].contiguous(), score[:, j].contiguous(),
                             None if ik is None else ik[:, j].contiguous(),
                             None if iks is None else iks[:, j].contiguous(), pos, **self._append_kw())

    def _kv_dtype(self):
        return torch.uint8 if self.kv8 else torch.bfloat16

    def _to_fp8(self, bf16_cache):
        """Quantise the bulk-built bf16 cache and window ring into their fp8 stores (once, untimed)."""
        codes = torch.empty(bf16_cache.shape, dtype=torch.uint8, device=self.dev)
        kv_quantize_fp8(bf16_cache, codes=codes, scales=self.kv_sc)
        kv_quantize_fp8(self._ring_bf16, codes=self.ring, scales=self.ring_sc)
        self._ring_bf16 = None
        return codes

    def _attend_kw(self):
        return dict(kv_scale=self.kv_sc, win_scale=self.ring_sc) if self.kv8 else {}

    def _window_and_proj_tail(self):
        if self.stack_h is not None:   # h <- h + layer(h), in place
            grouped_out_proj_residual(self.o.view(self.B, self.H * 512), self.w_g, self.w_o, self.stack_h, H=self.H,
                                      y=self.stack_h, ws=self.ws_proj)
            return
        grouped_out_proj(self.o.view(self.B, self.H * 512), self.w_g, self.w_o, H=self.H, y=self.y,
                         ws=self.ws_proj)

    def projection_segments(self):
        """(width, destination) of every input this layer takes from the hidden state, in the column
        order of its input-projection weights."""
        B = self.B
        segs = [(self.H * 512, self.q.view(B, self.H * 512)), (512, self.new_tok.view(B, 512)),
                (1, self.new_score.view(B))]
        if isinstance(self, CsaDecodeLayer):
            segs += [(self.H_I * self.dI, self.q_idx.view(B, self.H_I * self.dI)), (self.H_I, self.w_idx.view(B, self.H_I)),
                     (self.dI, self.new_ik), (1, self.new_is)]
        return segs


class CsaDecodeLayer(_Common):
    """One CSA layer (m = 4 with an overlap of 4, fp8 indexer 64 x 128, top-k k)."""

    def __init__(self, B, ctx, k=1024, H=64, H_I=64, dI=128, W=128, g=8, d_g=1024, d=4096, m=4, ov=4,
                 device="cuda", weights_std=0.02, seed=0, kv8=False):
        super().__init__(B, ctx, H, W, g, d_g, d, device, weights_std, seed, kv8)
        self.k, self.H_I, self.dI, self.m, self.ov = k, H_I, dI, m, ov
        self.n_cap = ctx // m
        nrm = self._nrm
        self.kv_cache = torch.empty((B, self.n_cap, 512), dtype=self._kv_dtype(), device=device)
        self.kv_sc = torch.empty((B, self.n_cap), dtype=torch.float32, device=device) if kv8 else None
        self.ik_cache = torch.empty((B, self.n_cap, dI), dtype=torch.uint8, device=device)
        self.ik_scale = torch.empty((B, self.n_cap), dtype=torch.float32, device=device)
        self.new_ik = nrm((B, dI), 1.28).to(torch.bfloat16)
        self.new_is = nrm((B,), 1.28)
        self.q_idx = nrm((B, 1, H_I, dI), 1.28).to(torch.bfloat16)
        self.w_idx = nrm((B, 1, H_I), 1.28).to(torch.bfloat16)
        self.topk = torch.empty((B, 1, k), dtype=torch.int32, device=device)
        self.ws_index = workspace(csa_index_topk_workspace(B, 1, self.n_cap, k), device, zeroed=True)
        self.ws_attn = workspace(attend_workspace(B, 1, H, k + W), device)

    def build_caches(self, block_tokens=65536, seed=1):
        """Fill the compressed caches for tokens [0, ctx) from seeded raw per-token data on the device,
        through csa_compress_kv (bulk path), and the window ring for tokens [ctx-W+1, ctx)."""
        B, m, ov = self.B, self.m, self.ov
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(seed)
        nb_per = block_tokens // m
        if self.kv8:                     # bulk path in bf16, then one quantisation pass
            self.kv_cache = torch.empty((B, self.n_cap, 512), dtype=torch.bfloat16, device=self.dev)
        for blk0 in range(0, self.n_cap, nb_per):
            nb = min(nb_per, self.n_cap - blk0)
            t0 = max(0, blk0 * m - ov)
            T = (blk0 + nb) * m - t0
            kv = torch.empty((B, T, 512), device=self.dev).normal_(0, 1.28, generator=gen).to(torch.bfloat16)
            ks = torch.empty((B, T), device=self.dev).normal_(0, 1.28, generator=gen)
            ik = torch.empty((B, T, self.dI), device=self.dev).normal_(0, 1.28, generator=gen).to(torch.bfloat16)
            iks = torch.empty((B, T), device=self.dev).normal_(0, 1.28, generator=gen)
            csa_compress_kv(kv, ks, ik, iks, tok0=t0, blk_begin=blk0, n_blk=nb, m=m, overlap=ov, gamma_kv=self.gamma,
                            kv_out=self.kv_cache, ik_out=self.ik_cache, ik_scale=self.ik_scale, ik_fp8=True)
            if blk0 + nb == self.n_cap:
                w0 = max(0, self.ctx - self.W + 1)
                self.fill_ring(kv[:, w0 - t0:].contiguous(), ks[:, w0 - t0:].contiguous(), w0)
                if self.kv8:
                    self.kv_cache = self._to_fp8(self.kv_cache)
                p0 = self.ctx - ov                # the open block at t = ctx starts ov tokens earlier
                self.prime(kv[:, p0 - t0:], ks[:, p0 - t0:], ik[:, p0 - t0:], iks[:, p0 - t0:], p0)
            del kv, ks, ik, iks

    def _append_kw(self):
        return dict(m=self.m, overlap=self.ov, gamma_kv=self.gamma, state=self.state, kv_out=self.kv_cache,
                    win=self.ring, ring_cap=RING, ik_out=self.ik_cache, ik_scale=self.ik_scale, ik_fp8=True,
                    kv_scale=self.kv_sc, win_scale=self.ring_sc)

    def step(self):
        # the token append runs inside the selection call (beside its final kernel): nothing the append
        # writes is read by this step's selection, and the attention after it sees the new ring row
        append = dict(kv_tok=self.new_tok.view(self.B, 512), kv_score=self.new_score.view(self.B), ik_tok=self.new_ik,
                      ik_score=self.new_is, pos=self.q_pos.view(self.B), **self._append_kw())
        csa_index_topk_append(self.q_idx, self.w_idx, self.ik_cache, self.ik_scale, self.q_pos, n_cap=self.n_cap,
                              m=self.m, k=self.k, topk_idx=self.topk, ws=self.ws_index, append=append)
        csa_attend(self.q, self.gamma, self.kv_cache, self.topk, self.ring, self.sink, self.q_pos, window=self.W,
                   ring_cap=RING, out=self.o, ws=self.ws_attn, **self._attend_kw())
        self._window_and_proj_tail()

    def bytes_per_step(self):
        """Algorithmic HBM bytes of one step (each key/entry/weight read once, outputs written once)."""
        B, k, W, H = self.B, self.k, self.W, self.H
        n_vis = min(self.t // self.m, self.n_cap)
        index = B * n_vis * (self.dI + 4) + B * self.H_I * (self.dI * 2 + 2)
        row = 516 if self.kv8 else 1024
        attend = B * (min(k, n_vis) + W) * row + B * H * 512 * 2 * 2 + B * k * 4
        proj = (self.w_g.numel() + self.w_o.numel()) * 2 + B * (H * 512 + self.d) * 2
        # append: token + key + logits read, ring row written, two pooling-state slots (read + write, write)
        slot = (512 + 128 + 8) * 4
        compress = B * ((512 + self.dI) * 2 + 8 + 512 * 2 + 3 * slot)
        return {"index": index, "attend": attend, "proj": proj, "compress": compress}


class HcaDecodeLayer(_Common):
    """One HCA layer (m' = 128, no overlap, dense attention over every visible entry)."""

    def __init__(self, B, ctx, H=64, W=128, g=8, d_g=1024, d=4096, m=128, device="cuda", weights_std=0.02, seed=0,
                 kv8=False):
        super().__init__(B, ctx, H, W, g, d_g, d, device, weights_std, seed, kv8)
        self.m = m
        self.n_cap = ctx // m
        self.kv_cache = torch.empty((B, self.n_cap, 512), dtype=self._kv_dtype(), device=device)
        self.kv_sc = torch.empty((B, self.n_cap), dtype=torch.float32, device=device) if kv8 else None
        self.ws_attn = workspace(attend_workspace(B, 1, H, self.n_cap + W), device)

    def build_caches(self, block_tokens=65536, seed=1):
        B, m = self.B, self.m
        gen = torch.Generator(device=self.dev)
        gen.manual_seed(seed)
        nb_per = block_tokens // m
        if self.kv8:                     # bulk path in bf16, then one quantisation pass
            self.kv_cache = torch.empty((B, self.n_cap, 512), dtype=torch.bfloat16, device=self.dev)
        for blk0 in range(0, self.n_cap, nb_per):
            nb = min(nb_per, self.n_cap - blk0)
            t0 = blk0 * m
            T = nb * m
            kv = torch.empty((B, T, 512), device=self.dev).normal_(0, 1.28, generator=gen).to(torch.bfloat16)
            ks = torch.empty((B, T), device=self.dev).normal_(0, 1.28, generator=gen)
            hca_compress_kv(kv, ks, tok0=t0, blk_begin=blk0, n_blk=nb, m=m, gamma_kv=self.gamma, kv_out=self.kv_cache)
            if blk0 + nb == self.n_cap:
                w0 = max(0, self.ctx - self.W + 1)
                self.fill_ring(kv[:, w0 - t0:].contiguous(), ks[:, w0 - t0:].contiguous(), w0)
                if self.kv8:
                    self.kv_cache = self._to_fp8(self.kv_cache)
            del kv, ks

    def _append_kw(self):
        return dict(m=self.m, overlap=0, gamma_kv=self.gamma, state=self.state, kv_out=self.kv_cache, win=self.ring,
                    ring_cap=RING, kv_scale=self.kv_sc, win_scale=self.ring_sc)

    def step(self):
        # the token append runs in the attention's launch; the query's own window row is formed by the
        # split that holds it, so nothing waits for the ring row the append writes
        append = dict(kv_tok=self.new_tok.view(self.B, 512), kv_score=self.new_score.view(self.B), ik_tok=None,
                      ik_score=None, pos=self.q_pos.view(self.B), **self._append_kw())
        hca_attend_append(self.q, self.gamma, self.sink, self.q_pos, n_cap=self.n_cap, window=self.W, out=self.o,
                          ws=self.ws_attn, append=append)
        self._window_and_proj_tail()

    def bytes_per_step(self):
        B, W, H = self.B, self.W, self.H
        n_vis = min(self.t // self.m, self.n_cap)
        row = 516 if self.kv8 else 1024
        attend = B * (n_vis + W) * row + B * H * 512 * 2 * 2
        proj = (self.w_g.numel() + self.w_o.numel()) * 2 + B * (H * 512 + self.d) * 2
        compress = B * (512 * 2 + 4 + 512 * 2 + (512 + 8) * 4)   # token + logit, ring row, state slot written
        return {"attend": attend, "proj": proj, "compress": compress}


def hybrid_stack(B=8, ctx=1 << 20, k=1024, device="cuda", build=True, kv8=False):
    """The 4-layer decode stack (CSA, HCA, CSA, HCA) at one GPU's share of the hybrid configuration
    (kv8: fp8 K=V storage)."""
    layers = []
    for i, kind in enumerate(("csa", "hca", "csa", "hca")):
        L = CsaDecodeLayer(B, ctx, k=k, device=device, seed=100 + i, kv8=kv8) if kind == "csa" else \
            HcaDecodeLayer(B, ctx, device=device, seed=100 + i, kv8=kv8)
        if build:
            L.build_caches(seed=200 + i)
        layers.append(L)
    return layers


def flops_per_step(layer):
    """Algorithmic flops: indexer dots (2 d_I per head-entry), QK^T + PV (4 c per head-key), projections."""
    B, H = layer.B, layer.H
    proj = 2 * B * (layer.w_g.numel() + layer.w_o.numel())
    if isinstance(layer, CsaDecodeLayer):
        n_vis = min(layer.t // layer.m, layer.n_cap)
        return {"index": 2 * B * n_vis * layer.H_I * layer.dI,
                "attend": 4 * 512 * B * H * (min(layer.k, n_vis) + layer.W), "proj": proj}
    n_vis = min(layer.t // layer.m, layer.n_cap)
    return {"attend": 4 * 512 * B * H * (n_vis + layer.W), "proj": proj}


class ChainedStack:
    """The decode stack as a chain: each layer's inputs (query heads, K=V token and logit, indexer
    query, head weights, key and logit) come from one input projection of the hidden state h [B, d],
    and each layer's grouped projection adds its output to h in place (h <- h + y).  h is reset from
    h0 at the start of every step, so repeated steps compute the same thing."""

    def __init__(self, layers, d=4096, weights_std=0.02, seed=7):
        self.layers = layers
        dev = layers[0].dev
        B = layers[0].B
        gen = torch.Generator(device=dev)
        gen.manual_seed(seed)
        self.h0 = torch.empty((B, d), device=dev).normal_(0.0, 1.0, generator=gen).to(torch.bfloat16)
        self.h = self.h0.clone()
        self.w_in, self.segs = [], []
        for layer in layers:
            segs = layer.projection_segments()
            n = sum(w for w, _ in segs)
            n_rows = (n + 15) // 16 * 16
            w = torch.empty((n_rows, d), device=dev).normal_(0.0, weights_std, generator=gen).to(torch.bfloat16)
            self.w_in.append(w)
            self.segs.append(segs)
            layer.stack_h = self.h

    def step(self):
        self.h.copy_(self.h0)
        for layer, w, segs in zip(self.layers, self.w_in, self.segs):
            input_proj(self.h, w, segs)
            layer.step()

    def proj_bytes(self):
        return sum(w.numel() * 2 for w in self.w_in) + len(self.layers) * self.h.numel() * 2 * 2


__all__ = ["CsaDecodeLayer", "HcaDecodeLayer", "ChainedStack", "hybrid_stack", "flops_per_step", "RING"]
_ = math
