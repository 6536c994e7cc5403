"""Exhaustive reference for GAC's rank selection.

TEST INFRASTRUCTURE ONLY (like the rest of ``oracle``): only the tests may
import it.  It shares no code with the library's dynamic program
(rank_linear_layer_amd/csrc/lr_gac.cpp).

"Why Smaller Is Slower? Dimensional Misalignment in Compressed LLMs",
section 4.3 (Step 3: Constrained Optimization): choose one dimension d_i
from each candidate set C_i to maximize

    sum_i s_i * (|W_i| - |W_i*|),   |W_i| = c_i d_i,  |W_i*| = c_i d*_i,

subject to sum_i |W_i| <= B, where c_i is the parameter cost of one
retained dimension.  With the page's budget quantization by a unit u, a
choice costs ceil(c_i d_i / u) units and the budget is floor(B / u) units.
This module enumerates every combination (small instances only).
"""
from __future__ import annotations

import itertools
from fractions import Fraction


def quantized_cost(c: int, d: int, u: int) -> int:
    return -((-c * d) // u)  # ceil(c d / u)


def best_selection(scores, unit_costs, d_star, cands, budget: int, unit: int):
    """(best objective, list of all optimal selections) over every
    combination whose quantized cost fits; None if nothing fits.
    Objectives are exact rationals (scores and d* as given, converted
    exactly)."""
    u = unit if unit > 0 else 8 * min(unit_costs)
    cap = budget // u
    best, arg = None, []
    for combo in itertools.product(*cands):
        cost = sum(quantized_cost(c, d, u) for c, d in zip(unit_costs, combo))
        if cost > cap:
            continue
        obj = sum(Fraction(s) * (Fraction(c * d) - Fraction(c) * Fraction(ds))
                  for s, c, d, ds in zip(scores, unit_costs, combo, d_star))
        if best is None or obj > best:
            best, arg = obj, [list(combo)]
        elif obj == best:
            arg.append(list(combo))
    if best is None:
        return None
    return best, arg
