"""CPU oracle for the factorized linear layer Y = (X.A).B.

TEST INFRASTRUCTURE ONLY: the oracle is what the GPU path is checked
against.  Only the test suite, the package smoke check and the benchmark's
CPU-baseline leg may import it.  The GPU library never calls it and shares no
code with it; the two meet only through the seeded inputs of
``rank_linear_layer_amd.datagen``.

Definition (plain product, float64, sequential sums, no FMA) -- see the
header of ``oracle.c``:
  "Why Smaller Is Slower? Dimensional Misalignment in Compressed LLMs",
  section 1 / Figure 1 (W replaced by A.B, rank r the inner dimension);
  "LowRankArena ...", Prerequisites, Figure A (y = Wx becomes y = A(Bx)).

Parity metrics (``rel_fro``, ``max_abs_ratio``) compare a bf16 GPU output,
decoded exactly, with the float64 oracle output.

Every function here is pinned by the CPU tests (tests/test_oracle.py) to
something other than itself: exact rational brute force, closed forms
(identity and rank-1 factors, the Eckart-Young-Mirsky error of a truncated
SVD), and the zero-padding invariance of the rank.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")
_lib = None
_lock = threading.Lock()


def build(force: bool = True) -> str:
    """Compile oracle.c with gcc (float64, -ffp-contract=off, OpenMP)."""
    if not force and os.path.exists(_LIB_PATH):
        return _LIB_PATH
    tmp = _LIB_PATH + ".tmp%d" % os.getpid()
    cmd = ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-fopenmp",
           "-ffp-contract=off", "-fno-fast-math", "-o", tmp, _SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


def _load():
    global _lib
    with _lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        P = ctypes.c_void_p
        I = ctypes.c_int64
        lib.oracle_lowrank_f64.argtypes = [P, P, P, I, I, I, I, P, P, ctypes.c_int]
        lib.oracle_lowrank_f64.restype = None
        lib.oracle_lowrank_bf16.argtypes = [P, P, P, I, I, I, I, P, ctypes.c_int]
        lib.oracle_lowrank_bf16.restype = ctypes.c_int
        lib.oracle_lowrank_bf16_sampled.argtypes = [P, P, P, I, I, I, I, P, I, P, I, P, ctypes.c_int]
        lib.oracle_lowrank_bf16_sampled.restype = ctypes.c_int
        lib.oracle_bf16_decode.argtypes = [P, P, I]
        lib.oracle_bf16_decode.restype = None
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib = lib
        return lib


def default_threads() -> int:
    try:
        return max(1, len(os.sched_getaffinity(0)))
    except AttributeError:  # pragma: no cover
        return max(1, os.cpu_count() or 1)


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a, a.ctypes.data_as(ctypes.c_void_p)


def _shapes(X, A, B):
    M, K = X.shape
    K2, r = A.shape
    r2, N = B.shape
    if K2 != K or r2 != r:
        raise ValueError("shape mismatch: X%s A%s B%s" % (X.shape, A.shape, B.shape))
    return M, K, r, N


def bf16_decode(bits) -> np.ndarray:
    """bf16 bit patterns -> float64 (exact), via the C decoder."""
    lib = _load()
    b, pb = _c(bits, np.uint16)
    out = np.empty(b.shape, dtype=np.float64)
    lib.oracle_bf16_decode(pb, out.ctypes.data_as(ctypes.c_void_p), b.size)
    return out


def lowrank_f64(X, A, B, nthreads: int | None = None) -> np.ndarray:
    """Y = (X.A).B with float64 inputs (sequential sums, no FMA)."""
    lib = _load()
    M, K, r, N = _shapes(np.asarray(X), np.asarray(A), np.asarray(B))
    X, pX = _c(X, np.float64)
    A, pA = _c(A, np.float64)
    B, pB = _c(B, np.float64)
    T = np.empty((M, r), dtype=np.float64)
    Y = np.empty((M, N), dtype=np.float64)
    lib.oracle_lowrank_f64(pX, pA, pB, M, K, r, N,
                           T.ctypes.data_as(ctypes.c_void_p),
                           Y.ctypes.data_as(ctypes.c_void_p),
                           nthreads or default_threads())
    return Y


def lowrank_bf16(Xb, Ab, Bb, nthreads: int | None = None) -> np.ndarray:
    """Y = (X.A).B in float64 from bf16 bit patterns (uint16 arrays)."""
    lib = _load()
    M, K, r, N = _shapes(np.asarray(Xb), np.asarray(Ab), np.asarray(Bb))
    Xb, pX = _c(Xb, np.uint16)
    Ab, pA = _c(Ab, np.uint16)
    Bb, pB = _c(Bb, np.uint16)
    Y = np.empty((M, N), dtype=np.float64)
    rc = lib.oracle_lowrank_bf16(pX, pA, pB, M, K, r, N,
                                 Y.ctypes.data_as(ctypes.c_void_p),
                                 nthreads or default_threads())
    if rc != 0:
        raise MemoryError("oracle_lowrank_bf16: allocation failed")
    return Y


def lowrank_bf16_sampled(Xb, Ab, Bb, rows, cols, nthreads: int | None = None) -> np.ndarray:
    """Y[rows][:, cols] of (X.A).B in float64, computed one output at a time."""
    lib = _load()
    M, K, r, N = _shapes(np.asarray(Xb), np.asarray(Ab), np.asarray(Bb))
    Xb, pX = _c(Xb, np.uint16)
    Ab, pA = _c(Ab, np.uint16)
    Bb, pB = _c(Bb, np.uint16)
    rows, pr = _c(rows, np.int64)
    cols, pc = _c(cols, np.int64)
    if rows.size and (rows.min() < 0 or rows.max() >= M):
        raise IndexError("row out of range")
    if cols.size and (cols.min() < 0 or cols.max() >= N):
        raise IndexError("col out of range")
    Y = np.empty((rows.size, cols.size), dtype=np.float64)
    rc = lib.oracle_lowrank_bf16_sampled(pX, pA, pB, M, K, r, N, pr, rows.size, pc, cols.size,
                                         Y.ctypes.data_as(ctypes.c_void_p),
                                         nthreads or default_threads())
    if rc != 0:
        raise MemoryError("oracle_lowrank_bf16_sampled: allocation failed")
    return Y


def lowrank_numpy_f64(X, A, B) -> np.ndarray:
    """Second, independent implementation: numpy BLAS (X @ A) @ B in float64."""
    return (np.asarray(X, np.float64) @ np.asarray(A, np.float64)) @ np.asarray(B, np.float64)


# ---------------------------------------------------------------- metrics ---

def rel_fro(y, y_ref) -> float:
    """||y - y_ref||_F / ||y_ref||_F (0 if both are zero, inf if only y_ref is)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = float(np.sqrt(np.sum(y_ref * y_ref)))
    num = float(np.sqrt(np.sum((y - y_ref) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def max_abs_ratio(y, y_ref) -> float:
    """max|y - y_ref| / max|y_ref| (0 if both are zero, inf if only y_ref is)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    if y_ref.size == 0:
        return 0.0
    den = float(np.max(np.abs(y_ref)))
    num = float(np.max(np.abs(y - y_ref)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


# Tolerances for a bf16-in / fp32-accumulate / bf16-out kernel.
REL_FRO_TOL = 5e-3
MAX_ABS_TOL = 2e-2


def parity(y_gpu_bits, y_ref) -> dict:
    """Compare bf16 output bits with the float64 oracle output."""
    y = bf16_decode(y_gpu_bits)
    rf = rel_fro(y, y_ref)
    ma = max_abs_ratio(y, y_ref)
    finite = bool(np.all(np.isfinite(y)))
    return {"rel_fro": rf, "max_abs": ma, "finite": finite,
            "ok": finite and rf <= REL_FRO_TOL and ma <= MAX_ABS_TOL}
