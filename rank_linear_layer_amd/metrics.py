"""Host-side accounting for the factorized linear layer: stored parameters,
keep ratio, algorithmic bytes and flops (used by the benchmark's roofline).

Parameter count of a rank-k factor pair of an m x n weight is k(m + n)
instead of mn ("LowRankArena ...", Prerequisites, Figure A).  The keep ratio
of a set of compressed layers sums stored parameters over all layers and
divides by the sum of dense parameters, at equal precision ("LowRankArena
...", "The standardized keep-ratio formula, expanded"); its worked example
(two layers, 4096x4096 at rank 1024 and 4096x11008 at rank 2048) gives
39,321,600 / 61,865,984.
"""
from __future__ import annotations

from fractions import Fraction
from typing import Iterable, Tuple

BF16_BYTES = 2


def lowrank_params(m: int, n: int, k: int) -> int:
    """Stored scalars of a rank-k factorization of an m x n weight."""
    return k * (m + n)


def dense_params(m: int, n: int) -> int:
    return m * n


def keep_ratio(layers: Iterable[Tuple[int, int, int]]) -> Fraction:
    """Exact keep ratio of layers given as (m, n, k) triples."""
    num = 0
    den = 0
    for m, n, k in layers:
        num += lowrank_params(m, n, k)
        den += dense_params(m, n)
    if den == 0:
        raise ValueError("no layers")
    return Fraction(num, den)


def decode_bytes(M: int, K: int, r: int, N: int) -> int:
    """Algorithmic HBM bytes of one factorized projection (bf16 X, A, B read
    once, bf16 Y written once; T stays on chip and is not counted)."""
    return BF16_BYTES * (M * K + K * r + r * N + M * N)


def lowrank_flops(M: int, K: int, r: int, N: int) -> int:
    """Algorithmic flops 2*M*r*(K + N) with the unpadded rank."""
    return 2 * M * r * (K + N)


def dense_bytes(M: int, K: int, N: int) -> int:
    return BF16_BYTES * (M * K + K * N + M * N)
