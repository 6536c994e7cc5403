"""GAC rank re-selection on MI355X ("Why Smaller Is Slower? Dimensional
Misalignment in Compressed LLMs", section 4: GAC, GPU-Aligned Compression).

Step 2 (Dimension Sweep, section 4.2) builds each weight's candidate set
from a latency table measured on this GPU; step 3 (Constrained
Optimization, section 4.3) is the dynamic program in the C library
(lr_gac_select, include/lr_gac.h).  Step 1, the compressor's continuous
allocation and importance scores, is an input.

    cands = [candidates(d, latency_of) for d in d_star]
    dims, obj = select(scores, unit_costs, d_star, cands, budget)
"""
from __future__ import annotations

import ctypes
import math

from . import _check, load_library

ALIGN = 8                # the heuristic filter: d mod 8 == 0 (the pages' minimum requirement)
WINDOW = (0.85, 1.20)    # candidates between 0.85 d* and 1.2 d*
TOL = 0.05               # a larger dimension must be over 5% faster to mark d as a cliff (timing noise)


def quantization_unit(unit_costs, align: int = ALIGN) -> int:
    """The page's budget quantum: align x the smallest per-dimension cost."""
    return align * min(int(c) for c in unit_costs)


def candidates(d_star: float, latency, align: int = ALIGN, window=WINDOW, tol: float = TOL):
    """Candidate dimensions for a continuous allocation d_star.

    Multiples of `align` in [window[0] d*, window[1] d*] (at least one
    multiple, the one nearest d*), minus the dimensions the sweep shows to
    sit on a cliff: d is dropped when a larger candidate runs faster than
    latency(d) / (1 + tol), since it keeps more parameters for less time.
    `latency` maps a dimension to its measured time (a dict or a callable).
    """
    lat = latency.get if isinstance(latency, dict) else latency
    lo = max(align, int(math.ceil(window[0] * d_star / align)) * align)
    hi = int(math.floor(window[1] * d_star / align)) * align
    dims = list(range(lo, hi + 1, align))
    if not dims:
        dims = [max(align, int(round(d_star / align)) * align)]
    times = {d: lat(d) for d in dims}
    keep = []
    for i, d in enumerate(dims):
        if times[d] is None:
            continue
        faster_larger = any(times[e] is not None and times[e] * (1.0 + tol) < times[d] for e in dims[i + 1:])
        if not faster_larger:
            keep.append(d)
    return keep


def select(scores, unit_costs, d_star, cands, budget: int, unit: int = 0):
    """One dimension per weight maximizing sum s_i c_i (d_i - d*_i) with
    sum c_i d_i <= budget (costs quantized by `unit`, 0 = 8 min c_i).
    Returns (dims, objective)."""
    n = len(scores)
    if not (len(unit_costs) == len(d_star) == len(cands) == n):
        raise ValueError("scores, unit_costs, d_star and cands must have one entry per weight")
    dbl, i64, cint = ctypes.c_double, ctypes.c_int64, ctypes.c_int
    flat = [int(d) for c in cands for d in c]
    out = (i64 * max(n, 1))()
    obj = dbl(0.0)
    st = load_library().lr_gac_select(
        n, (dbl * max(n, 1))(*[float(s) for s in scores]), (i64 * max(n, 1))(*[int(c) for c in unit_costs]),
        (dbl * max(n, 1))(*[float(d) for d in d_star]), (cint * max(n, 1))(*[len(c) for c in cands]),
        (i64 * max(len(flat), 1))(*flat), int(budget), int(unit), out, ctypes.byref(obj))
    _check(st, "lr_gac_select")
    return [int(out[i]) for i in range(n)], float(obj.value)
