"""Seeded synthetic inputs for the factorized linear layer Y = (X.A).B.

This module is shared by the GPU path's tests/bench and by the CPU oracle's
tests. It only *draws* inputs; it holds none of the layer's arithmetic.

Distributions follow the workloads of the low-rank pages: activations
X ~ N(0, 1); factors A[K x r] ~ N(0, std = 1/sqrt(K)) and B[r x N] ~
N(0, std = 1/sqrt(r)) ("fan_in" of each factor), so that T = X.A and Y have
unit RMS.  Every draw uses numpy's PCG64 generator in float64, is scaled,
cast to float32 and then rounded to bfloat16 with round-to-nearest-even.
Arrays are returned as uint16 bit patterns, row-major and contiguous.

A second generator builds factor pairs the way SVD compression does
("LowRankArena ...", Prerequisites, Figure A): A = U[:, :k] S^(1/2),
B = S^(1/2) V[:, :k]^T from the SVD of a seeded Gaussian matrix.  That is an
*input recipe* (structured factors), not part of Y = (X.A).B.
"""
from __future__ import annotations

import numpy as np

__all__ = [
    "bf16_bits_from_f32",
    "bf16_bits_to_f32",
    "normal_bf16",
    "factorized_inputs",
    "svd_factor_inputs",
    "gaussian_matrix_f64",
]


def bf16_bits_from_f32(x) -> np.ndarray:
    """float32 -> bfloat16 bit patterns, round-to-nearest-even on the
    16 dropped mantissa bits.  Inputs must be finite (generators never
    produce inf/nan)."""
    x = np.ascontiguousarray(np.asarray(x, dtype=np.float32))
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> np.uint64(16)) & np.uint64(1)
    rounded = (u + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return rounded.astype(np.uint16)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """bfloat16 bit patterns -> float32 (exact)."""
    b = np.ascontiguousarray(np.asarray(bits, dtype=np.uint16))
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32)


def normal_bf16(shape, std: float, seed: int) -> np.ndarray:
    """N(0, std^2) draws rounded to bf16, returned as uint16 bits."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    x = rng.standard_normal(size=shape, dtype=np.float64)
    if std != 1.0:
        x *= std
    return bf16_bits_from_f32(x.astype(np.float32))


def factorized_inputs(M: int, K: int, r: int, N: int, seed_base: int):
    """(X, A, B) bf16 bit arrays for one factorized projection.

    Seeds: X <- seed_base + 0, A <- seed_base + 1, B <- seed_base + 2.
    """
    X = normal_bf16((M, K), 1.0, seed_base + 0)
    A = normal_bf16((K, r), 1.0 / np.sqrt(K), seed_base + 1)
    B = normal_bf16((r, N), 1.0 / np.sqrt(r), seed_base + 2)
    return X, A, B


def gaussian_matrix_f64(rows: int, cols: int, seed: int) -> np.ndarray:
    """Seeded N(0,1) float64 matrix (the dense weight W of the SVD recipe)."""
    rng = np.random.Generator(np.random.PCG64(int(seed)))
    return rng.standard_normal(size=(rows, cols), dtype=np.float64)


def svd_factor_inputs(K: int, N: int, k: int, seed: int):
    """Factor pair of the rank-k truncated SVD of a seeded Gaussian W[K x N].

    Returns (W, A64, B64, A_bits, B_bits): the float64 matrix, the float64
    factors A = U[:, :k] sqrt(S[:k]) (K x k) and B = sqrt(S[:k]) V[:, :k]^T
    (k x N), and their bf16 bit patterns (what a bf16 kernel consumes).
    """
    W = gaussian_matrix_f64(K, N, seed)
    U, S, Vt = np.linalg.svd(W, full_matrices=False)
    root = np.sqrt(S[:k])
    A64 = U[:, :k] * root[None, :]
    B64 = root[:, None] * Vt[:k, :]
    A_bits = bf16_bits_from_f32(A64.astype(np.float32))
    B_bits = bf16_bits_from_f32(B64.astype(np.float32))
    return W, np.ascontiguousarray(A64), np.ascontiguousarray(B64), A_bits, B_bits
