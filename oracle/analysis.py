"""Closed forms from the LazyAttention paper -- TEST INFRASTRUCTURE ONLY.

Hit-ratio model (§2, Eqs. 1-3) and the per-tile cost model of deferred
rotation (§3.1 "Naive deferred encoding is expensive", §3.2 Eqs. 5-6).
Each function is written from the quantity's definition (FLOP or element
counts per tile), not from the simplified ratio, so that the printed
percentages in the pages check the reading of M, N and D.

Pins: tests/golden/paper_figures.json holds the pages' printed values
(2.86x, 150 %, 1.17 %, ~100 %, 0.59 %, 3.1 %, 1.17 %); Hurwitz-zeta partial
sums from scipy check the Zipf sums for alpha > 1.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "zipf_partial_sum",
    "hit_ratio_agnostic",
    "hit_ratio_aware",
    "hit_ratio_gap",
    "naive_flops_overhead",
    "naive_io_overhead",
    "prefill_flops_overhead",
    "prefill_table_bandwidth",
    "decode_trigger_overhead",
    "decode_overhead",
]


def zipf_partial_sum(n: int, alpha: float) -> float:
    """sum_{i=1..n} i^-alpha (0 for n <= 0)."""
    if n <= 0:
        return 0.0
    i = np.arange(1, int(n) + 1, dtype=np.float64)
    return float(np.sum(i ** (-float(alpha))))


def hit_ratio_agnostic(C: int, N: int, alpha: float) -> float:
    """Eq. 1: a position-agnostic cache of C entries holds the top-C documents."""
    return zipf_partial_sum(min(C, N), alpha) / zipf_partial_sum(N, alpha)


def hit_ratio_aware(C: int, D: int, N: int, alpha: float) -> float:
    """Eq. 2: with D positional variants per document only floor(C/D) documents fit."""
    return zipf_partial_sum(min(C // D, N), alpha) / zipf_partial_sum(N, alpha)


def hit_ratio_gap(C: int, D: int, alpha: float) -> float:
    """Eq. 3: ratio of Eq. 1 to Eq. 2 (the pool size N cancels)."""
    return zipf_partial_sum(C, alpha) / zipf_partial_sum(C // D, alpha)


# Cost model of one (Q tile, K/V tile) pair: Q tile M x D, K/V tiles N x D.
def _gemm_flops(M, N, D):
    # Q K^T and P V, multiply and add counted as two FLOPs each.
    return 2 * (2 * M * N * D)


def _rotation_flops(rows, D):
    # A 2-D rotation per feature pair: 4 multiplies + 2 adds per pair.
    return (D // 2) * 6 * rows


def naive_flops_overhead(M: int, N: int = 16, D: int = 128) -> float:
    """Rotate every K tile twice (back to 0, then forward) per tile pair."""
    return 2 * _rotation_flops(N, D) / _gemm_flops(M, N, D)


def naive_io_overhead(M: int, N: int) -> float:
    """Two cos/sin vectors per K token, against reading Q, K and V tiles."""
    D = 1  # cancels
    extra = 2 * N * D
    return extra / (M * D + 2 * N * D)


def prefill_flops_overhead(M: int, N: int = 16, D: int = 128) -> float:
    """Eq. 5: one relative rotation of the K tile per tile pair."""
    return _rotation_flops(N, D) / _gemm_flops(M, N, D)


def prefill_table_bandwidth(N: int, D: int = 128) -> float:
    """One D-length cos/sin row per document against the K and V tiles (N x D each)."""
    return D / (2 * D * N)


def decode_trigger_overhead(N: int, D: int = 128) -> float:
    """Rotating the (M=1) q tile once, against one tile pair's GEMM FLOPs."""
    return _rotation_flops(1, D) / _gemm_flops(1, N, D)


def decode_overhead(B: int, N: int, D: int = 128) -> float:
    """Eq. 6: the per-trigger overhead times the fraction r = 1/B of tiles that trigger."""
    return (1.0 / B) * decode_trigger_overhead(N, D)

