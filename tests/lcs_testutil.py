"""Comparison helpers shared by the parity tests (no method arithmetic beyond what the oracle does).

Tolerances (bf16 outputs, from the stated parity bar): the maximum absolute error, taken relative to
max(1, rms(reference)) so that bf16 rounding of outputs larger than 1 is not counted against the
kernel, must be <= 2e-2, and the relative L2 error <= 5e-3.  fp8-indexer outputs compared with an
oracle that does not quantise the indexer: relative L2 <= 5e-2.
"""
from __future__ import annotations

import numpy as np

import oracle as O
import synth

MAX_ABS = 2e-2
REL_L2 = 5e-3
REL_L2_FP8_VS_EXACT = 5e-2


def to_np_bf16(t):
    """bf16 torch tensor (any device) -> float64 numpy, exactly."""
    import torch
    return synth.bf16_bits_to_f64(t.detach().cpu().contiguous().view(torch.int16).numpy().view(np.uint16))


def from_bits(bits, device="cuda"):
    """uint16 bf16 patterns (numpy) -> torch bfloat16 tensor on device."""
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def errors(got, ref, absolute=False):
    """(max-abs error, relative L2 error).  The max-abs error is taken relative to max(1, rms(ref)):
    for outputs of magnitude <= 1 (attention outputs) it is the absolute error; for larger ones
    (projection outputs, residual sums of rms ~ 5) it discounts the bf16 storage of the result itself,
    whose rounding alone is up to 2^-9 of each element.  absolute=True also returns the plain max-abs."""
    got = np.asarray(got, dtype=np.float64)
    ref = np.asarray(ref, dtype=np.float64)
    d = got - ref
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    abs_max = float(np.max(np.abs(d))) if d.size else 0.0
    max_abs = abs_max / max(1.0, rms)
    rel = float(np.linalg.norm(d) / max(np.linalg.norm(ref), 1e-30)) if d.size else 0.0
    return (max_abs, rel, abs_max) if absolute else (max_abs, rel)


def assert_close(got, ref, what, max_abs=MAX_ABS, rel_l2=REL_L2):
    ma, rl, am = errors(got, ref, absolute=True)
    assert ma <= max_abs and rl <= rel_l2, \
        f"{what}: max-abs {ma:.3e} (<= {max_abs}; absolute {am:.3e}), rel-L2 {rl:.3e} (<= {rel_l2})"
    return ma, rl


def check_topk_row(gpu_idx, oracle_scores, k, bound):
    """Validate one GPU top-k row against the oracle's float64 scores of the same inputs.

    gpu_idx [k] int (ascending, -1 padded); oracle_scores [n_vis]; bound [n_vis] = per-entry fp32
    accumulation error bound.  Sets must agree wherever the score gap to the k-th exceeds the bound.
    Returns the number of entries that differ inside the band.
    """
    n = oracle_scores.shape[0]
    want = min(k, n)
    g = np.asarray(gpu_idx)
    valid = g[g >= 0]
    assert valid.shape[0] == want, f"selected {valid.shape[0]} entries, expected {want}"
    assert np.all(g[want:] == -1), "padding must be -1"
    assert np.all(np.diff(valid) > 0), "indices must be strictly ascending"
    assert valid.size == 0 or (valid.min() >= 0 and valid.max() < n), "index out of the visible range"
    if want == 0:
        return 0
    ref = O.topk_select(oracle_scores, k)
    ref = ref[ref >= 0]
    if np.array_equal(ref, valid):
        return 0
    order = np.lexsort((np.arange(n), -oracle_scores))
    kth = oracle_scores[order[want - 1]]
    extra = np.setdiff1d(valid, ref)        # chosen by the GPU, not by the oracle
    missing = np.setdiff1d(ref, valid)      # chosen by the oracle, not by the GPU
    tau = 1e-6 * max(1.0, abs(kth))
    for s in extra:
        assert oracle_scores[s] >= kth - max(tau, bound[s]), f"GPU picked {s}: {oracle_scores[s]} vs kth {kth}"
    for s in missing:
        assert oracle_scores[s] <= kth + max(tau, bound[s]), f"GPU dropped {s}: {oracle_scores[s]} vs kth {kth}"
    return int(extra.size)


def index_oracle_row(q_idx_bits, w_idx_bits, k_deq, fp8, split=False):
    """Oracle scores for one query row (inputs as given to the GPU) and their fp32 error bounds.

    q_idx_bits [H_I, dI] bf16 patterns; w_idx_bits [H_I]; k_deq [n, dI] float64 dequantised keys.
    In fp8 mode the query rows are quantised with the kernel's fp32 decision rule.

    Bound of sum_h w_h relu(a_h) evaluated head by head in fp32: (2 dI + H + 8) 2^-23 mag,
    mag = sum_h |w_h| sum_d |q_hd k_d|.  The dI term is twice one fp32 unit in the last place per
    product: the matrix instructions' internal accumulation (order, width, rounding) is not that of
    round-to-nearest fp32 additions, and with few heads its error was seen to exceed dI 2^-23 mag.
    split=True: the evaluation the fp8 prefill scorer uses, sum_h (w_h/2)|a_h| + u.k with u = sum_h (w_h/2) q_h carried as 4 E4M3 parts.  Its |a| half has the
    bound above; its linear half adds an fp32 accumulation over 4 parts of dI products,
    (dI + 12) 2^-23 sum_d |u_d k_d| <= (dI + 12) 2^-23 mag / 2, plus one final addition, and the
    parts' remainder, 2^-19 max_d |u_d| sum_d |k_d|.
    """
    q = synth.bf16_bits_to_f64(q_idx_bits)
    w = synth.bf16_bits_to_f64(w_idx_bits)
    if fp8:
        _, _, q = O.fp8_quantize_rows(q, kernel_fp32=True)
    sc = O.index_scores(q, w, k_deq)
    mag = (np.abs(k_deq) @ np.abs(q).T) @ np.abs(w)
    H, dI = q.shape
    bound = mag * (2 * dI + H + 8) * 2.0 ** -23
    if split:
        u = 0.5 * (w[:, None] * q).sum(0)
        bound = bound + mag * ((dI + 12) / 2 + 2) * 2.0 ** -23 + np.abs(u).max() * np.abs(k_deq).sum(1) * 2.0 ** -19
    return sc, bound
