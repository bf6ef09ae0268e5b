"""Seeded synthetic inputs for the CSA/HCA attention forward.

This module is shared by the CPU oracle's tests, the GPU parity tests and the
benchmark.  It holds random-number plumbing, storage-format conversions
(IEEE fp32 <-> bfloat16 bit patterns) and the workload shapes, and nothing of
the method's own arithmetic: no pooling, normalisation, rotation, scoring,
selection, attention or projection lives here.

Seeding: host tensors come from ``numpy.random.Generator(PCG64(SeedSequence(
[1000 + cfg, tensor_id])))``, drawn in float32 and rounded to bfloat16 with
round-to-nearest-even.  Large caches are drawn on the device with a seeded
``torch.Generator`` (see :func:`device_normal_bf16`).
"""
from __future__ import annotations

import numpy as np

from .configs import CONFIGS, Workload, small_workload  # noqa: F401


def rng(cfg: int, tensor_id: int) -> np.random.Generator:
    """Independent, reproducible stream for one tensor of one workload."""
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([1000 + cfg, tensor_id])))


def f32_to_bf16_bits(x) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(np.asarray(x, dtype=np.float32)).view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    r = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b) -> np.ndarray:
    """Widen bfloat16 bit patterns (uint16) to float32 exactly."""
    b = np.ascontiguousarray(np.asarray(b, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def bf16_bits_to_f64(b) -> np.ndarray:
    return bf16_bits_to_f32(b).astype(np.float64)


def normal_bf16(shape, std: float, cfg: int, tensor_id: int, mean: float = 0.0) -> np.ndarray:
    """N(mean, std^2) drawn in float32, stored as bfloat16 bit patterns (uint16)."""
    x = rng(cfg, tensor_id).standard_normal(size=shape, dtype=np.float32) * np.float32(std)
    if mean:
        x = x + np.float32(mean)
    return f32_to_bf16_bits(x)


def normal_f32(shape, std: float, cfg: int, tensor_id: int) -> np.ndarray:
    return (rng(cfg, tensor_id).standard_normal(size=shape, dtype=np.float32) * np.float32(std))


def fp8_codes(shape, cfg: int, tensor_id: int) -> np.ndarray:
    """Uniformly random *finite* OCP E4M3FN byte codes (0x7F and 0xFF, the NaNs, excluded).

    Stands in for a quantised indexer-key cache: any finite code is a valid
    stored value, so index/top-k parity can be driven without running the
    quantiser that produces them.
    """
    g = rng(cfg, tensor_id)
    mag = g.integers(0, 127, size=shape, dtype=np.int64)        # 0..126 are finite magnitudes
    sign = g.integers(0, 2, size=shape, dtype=np.int64) << 7
    return (mag | sign).astype(np.uint8)


def positive_scales(shape, cfg: int, tensor_id: int) -> np.ndarray:
    """Positive per-row float32 scales of the size absmax/448 gives for N(0, 1.6) rows."""
    g = rng(cfg, tensor_id)
    return (np.float32(1.0 / 448.0) * (np.float32(2.0) + np.abs(g.standard_normal(size=shape, dtype=np.float32)))).astype(np.float32)


def device_normal_bf16(shape, std: float, seed: int, device="cuda"):
    """Large N(0, std^2) bfloat16 tensor drawn on the device with a seeded torch.Generator."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, float(std), generator=gen)
    return x.to(torch.bfloat16)


def device_normal_f32(shape, std: float, seed: int, device="cuda"):
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    x = torch.empty(shape, dtype=torch.float32, device=device)
    x.normal_(0.0, float(std), generator=gen)
    return x


def device_fp8_codes(shape, seed: int, device="cuda"):
    """Random finite E4M3FN codes drawn on the device (uint8 tensor)."""
    import torch
    gen = torch.Generator(device=device)
    gen.manual_seed(int(seed))
    mag = torch.randint(0, 127, shape, generator=gen, device=device, dtype=torch.int32)
    sign = torch.randint(0, 2, shape, generator=gen, device=device, dtype=torch.int32) * 128
    return (mag + sign).to(torch.uint8)
