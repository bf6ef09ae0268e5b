"""Workload shapes for the CSA/HCA attention forward.

The five named workloads follow the configurations this method is measured on
(the DeepSeek-V4 Flash setting on page 4, section 3.1: m = 4, 64 indexer heads
of dim 128, top-k 512, m' = 128; page 1, "hybrid attention": head dim 512,
RoPE on the last 64 dims, a 128-token window, a sink per head, grouped output
projection; top-k 1024 at 1M context).  Only shapes and distributions live here.
"""
from __future__ import annotations

import dataclasses
import math


@dataclasses.dataclass(frozen=True)
class Workload:
    name: str
    kind: str              # csa_prefill | hca_decode | csa_decode | csa_chunked_prefill | hybrid_decode
    cfg: int               # seed family
    B: int
    ctx: int               # tokens already in the sequence before the queries (decode: query t = ctx)
    Tq: int                # query tokens per sequence
    H: int = 64
    c: int = 512
    W: int = 128
    m: int = 4
    ov: int = 4
    m_hca: int = 128
    H_I: int = 64
    d_I: int = 128
    k: int = 512
    ik_fp8: bool = True
    d: int = 4096
    g: int = 8
    d_g: int = 1024
    std_tok: float = math.sqrt(4096 * 0.02 ** 2)   # std of a projection of N(0,1) hidden states
    std_w: float = 0.02
    sink_std: float = 1.0                            # 0 -> all sinks 0
    eps: float = 1e-6
    theta: float = 10000.0

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.c)

    def q_positions(self):
        """Absolute token index of every query (same for each sequence)."""
        if self.kind in ("csa_prefill",):
            return list(range(self.Tq))
        if self.kind == "csa_chunked_prefill":
            return list(range(self.ctx - self.Tq, self.ctx))
        return [self.ctx + i for i in range(self.Tq)]


CONFIGS = {w.name: w for w in (
    # single CSA layer, causal prefill, ctx 2048, d = 1024, H = 8, indexer 8 x 64 bf16, top-k 128, sink 0
    Workload("csa_prefill_2k", "csa_prefill", 1, B=1, ctx=2048, Tq=2048, H=8, H_I=8, d_I=64, k=128,
             ik_fp8=False, d=1024, std_tok=1.0, sink_std=0.0),
    # single HCA layer decode, B = 64, ctx 65536 -> 512 entries, H = 64
    Workload("hca_decode_64k", "hca_decode", 2, B=64, ctx=65536, Tq=1),
    # single CSA layer decode (Flash): B = 32, ctx 131072 -> 32768 entries, fp8 indexer 64 x 128, top-k 512
    Workload("csa_decode_128k", "csa_decode", 3, B=32, ctx=131072, Tq=1, k=512),
    # CSA chunked prefill: 4096 queries against a 1,048,576-token cache, top-k 1024, inputs N(0,1)
    Workload("csa_chunked_prefill_1m", "csa_chunked_prefill", 4, B=1, ctx=1 << 20, Tq=4096, k=1024,
             std_tok=1.0),
    # hybrid 4-layer decode (CSA, HCA, CSA, HCA) at 1M ctx, B = 8, top-k 1024, g = 8, d_g = 1024, d = 4096
    Workload("hybrid4_decode_1m", "hybrid_decode", 5, B=8, ctx=1 << 20, Tq=1, k=1024),
)}


def small_workload(kind: str, **kw) -> Workload:
    """Small shapes the oracle finishes in seconds that still span several tiles and a ragged tail."""
    base = dict(cfg=100, B=2, ctx=333, Tq=1, H=64, k=64, H_I=64, d_I=128, ik_fp8=True, W=128)
    base.update(kw)
    return Workload(name=f"small_{kind}", kind=kind, **base)
