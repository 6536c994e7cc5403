"""CPU tests of GAC rank re-selection ("Why Smaller Is Slower? Dimensional
Misalignment in Compressed LLMs", section 4): the library's dynamic program
(lr_gac_select) against exhaustive enumeration (oracle/gac.py) on small
instances, the page's worked numbers, closed forms, and the candidate
filter of the dimension sweep."""
import os
import random

import pytest

import rank_linear_layer_amd as lrl
from oracle import gac as ref

pytestmark = pytest.mark.skipif(not os.path.exists(lrl.LIB_PATH), reason="library not built")


def _gac():
    from rank_linear_layer_amd import gac
    return gac


def _check_against_bruteforce(scores, costs, dstar, cands, budget, unit):
    gac = _gac()
    want = ref.best_selection(scores, costs, dstar, cands, budget, unit)
    if want is None:
        with pytest.raises(lrl.LRError) as e:
            gac.select(scores, costs, dstar, cands, budget, unit)
        assert e.value.status == lrl.LR_ERR_INVALID_ARG
        return
    best, optimal = want
    dims, obj = gac.select(scores, costs, dstar, cands, budget, unit)
    # several selections can tie: the value is unique, the selection must be
    # one of the optimal ones and fit the quantized budget
    assert dims in optimal, (dims, optimal)
    assert obj == pytest.approx(float(best), rel=1e-12, abs=1e-9)
    u = unit if unit > 0 else 8 * min(costs)
    assert sum(ref.quantized_cost(c, d, u) for c, d in zip(costs, dims)) <= budget // u
    assert sum(c * d for c, d in zip(costs, dims)) <= budget


def test_dp_matches_exhaustive_search_on_random_instances():
    rng = random.Random(20260)
    for trial in range(300):
        n = rng.randint(1, 5)
        costs = [rng.choice([1, 3, 8, 17, 64, 100]) for _ in range(n)]
        dstar = [rng.uniform(1, 60) for _ in range(n)]
        cands = [sorted(rng.sample(range(0, 72, rng.choice([1, 4, 8])), rng.randint(1, 4))) for _ in range(n)]
        scores = [rng.choice([0.0, 0.5, 1.0, 2.5, -1.0, rng.uniform(0, 3)]) for _ in range(n)]
        total_max = sum(c * max(cs) for c, cs in zip(costs, cands))
        budget = rng.randint(0, total_max + 10)
        unit = rng.choice([0, 1, 1, 7, 16])
        _check_against_bruteforce(scores, costs, dstar, cands, budget, unit)


def test_exact_when_unit_is_one():
    # u = 1: the table is the exact knapsack; a budget one short of the
    # best combination forces the next one
    costs, dstar, scores = [3, 5], [10.0, 10.0], [1.0, 2.0]
    cands = [[8, 10, 12], [8, 10, 12]]
    gac = _gac()
    assert gac.select(scores, costs, dstar, cands, 3 * 12 + 5 * 12, 1)[0] == [12, 12]
    assert gac.select(scores, costs, dstar, cands, 3 * 12 + 5 * 12 - 1, 1)[0] == [10, 12]
    _check_against_bruteforce(scores, costs, dstar, cands, 3 * 12 + 5 * 12 - 1, 1)


def test_closed_forms():
    gac = _gac()
    # one weight, ample budget, positive score: the largest candidate
    assert gac.select([1.0], [100], [50.0], [[40, 48, 56, 64]], 10 ** 6)[0] == [64]
    # negative score: the smallest
    assert gac.select([-1.0], [100], [50.0], [[40, 48, 56, 64]], 10 ** 6)[0] == [40]
    # zero score: every choice is worth 0; the cheapest wins the tie
    dims, obj = gac.select([0.0], [100], [50.0], [[48, 40, 64]], 10 ** 6)
    assert dims == [40] and obj == 0.0
    # objective = s c (d - d*)
    dims, obj = gac.select([2.0], [10], [45.5], [[48]], 10 ** 6, 1)
    assert dims == [48] and obj == pytest.approx(2.0 * 10 * (48 - 45.5))
    # nothing fits: rejected
    with pytest.raises(lrl.LRError):
        gac.select([1.0], [100], [50.0], [[40]], 100 * 40 - 1, 1)


def test_budget_quantization_worked_example():
    # the page's example: 100 weights of 1024 x 1024 at rho = 15% give a raw
    # budget of 0.85 * 100 * 1024^2 (about 1e8 table entries); with
    # dimensions in multiples of 8 the unit is 8 * M_min = 8 * 1024
    gac = _gac()
    budget = 85 * 1024 * 1024  # 0.85 * 100 * 1024^2
    assert budget == 89128960
    u = gac.quantization_unit([1024] * 100)
    assert u == 8192
    assert budget // u == 10880
    # the quantized program over those 100 pruned weights (cost 1024 per
    # kept column) runs in the library: every weight at d* = 870.4 keeps
    # 85% of its 1024 columns; aligned candidates around it
    dstar = [0.85 * 1024] * 100
    cands = [[856, 864, 872, 880]] * 100
    dims, obj = gac.select([1.0] * 100, [1024] * 100, dstar, cands, budget)
    assert sum(1024 * d for d in dims) <= budget
    # 100 x 870.4 columns fit exactly: the best aligned choice keeps 87040
    # columns' worth, i.e. a mix of 864 and 872 (and 880/856 pairs) summing to
    # at most 87040
    assert sum(dims) <= 87040 and sum(dims) >= 87040 - 8


def test_candidate_filter_of_the_sweep():
    gac = _gac()
    # the page's example: d* = 107.3 -> 107 is not a candidate (misaligned),
    # 104 and 112 are
    flat = {d: float(d) for d in range(1, 400)}
    c = gac.candidates(107.3, flat)
    assert 107 not in c and 104 in c and 112 in c
    assert all(d % 8 == 0 for d in c)
    assert min(c) >= 0.85 * 107.3 and max(c) <= 1.2 * 107.3
    # a measured cliff: 120 is slower than 128, so 120 is dropped
    cliff = dict(flat)
    cliff[120] = 200.0
    c2 = gac.candidates(107.3, cliff)
    assert 120 not in c2 and 128 in c2 and 112 in c2
    # latency that only grows with d (no cliff, as on these kernels): every
    # aligned dimension in the window stays
    assert c == [d for d in range(96, 129, 8)]


def test_page_candidate_set_end_to_end():
    # The page's candidate set for d* = 107.3 (section 4.2: C = {96, 104,
    # 112, 128}) for two weights of equal cost c, budget = both weights at
    # d* (214.6 c, so d1 + d2 <= 214) and scores 2 and 1.  By hand: the
    # pairs that fit are those with d1 + d2 <= 214; the objective
    # sum_i s_i c (d_i - 107.3) is largest for (112, 96): 2 (4.7) - 11.3 =
    # -1.9 per c, against (104, 104): -9.9, (96, 112): -17.9, (104, 96):
    # -23.2.  Exhaustive search and the library agree with that.
    gac = _gac()
    C = [96, 104, 112, 128]
    c = 4096
    scores, costs, dstar = [2.0, 1.0], [c, c], [107.3, 107.3]
    budget = int(c * 214.6)
    best, optimal = ref.best_selection(scores, costs, dstar, [C, C], budget, c)
    assert optimal == [[112, 96]]
    assert float(best) == pytest.approx(c * (2 * 4.7 - 11.3), rel=1e-12)
    dims, obj = gac.select(scores, costs, dstar, [C, C], budget, c)
    assert dims == [112, 96] and obj == pytest.approx(float(best), rel=1e-12)
    # with equal scores the objective is c (d1 + d2 - 214.6): every pair
    # summing to 208 ties, and the library returns one of them
    best2, optimal2 = ref.best_selection([1.0, 1.0], costs, dstar, [C, C], budget, c)
    assert sorted(optimal2) == [[96, 112], [104, 104], [112, 96]]
    dims2, _ = gac.select([1.0, 1.0], costs, dstar, [C, C], budget, c)
    assert dims2 in optimal2


def test_layer_scale_instance_beats_rounding_down():
    # 32 layers x 7 projections of the Llama-3-8B-shaped layer at 15%
    # compression: the program's choice fits the budget and keeps at least
    # as much weighted value as rounding every d* down to a multiple of 8
    gac = _gac()
    shapes = [(4096, 4096), (4096, 1024), (4096, 1024), (4096, 4096), (4096, 14336), (4096, 14336), (14336, 4096)]
    rng = random.Random(7)
    scores, costs, dstar, cands = [], [], [], []
    for layer in range(32):
        for K, N in shapes:
            full = K * N / (K + N)
            d = 0.85 * full * rng.uniform(0.7, 1.0)
            scores.append(rng.uniform(0.5, 2.0))
            costs.append(K + N)
            dstar.append(d)
            cands.append(gac.candidates(d, lambda x: float(x)))
    budget = int(sum(c * d for c, d in zip(costs, dstar)))
    dims, obj = gac.select(scores, costs, dstar, cands, budget)
    assert sum(c * d for c, d in zip(costs, dims)) <= budget
    down = [int(d // 8) * 8 for d in dstar]
    obj_down = sum(s * c * (d - ds) for s, c, d, ds in zip(scores, costs, down, dstar))
    assert obj >= obj_down - 1e-6 * abs(obj_down)


def test_argument_errors():
    import ctypes
    lib = lrl.load_library()
    assert lib.lr_gac_select(0, None, None, None, None, None, 0, 0, None, None) == lrl.LR_ERR_INVALID_ARG
    gac = _gac()
    with pytest.raises(lrl.LRError):
        gac.select([1.0], [0], [5.0], [[8]], 100)       # unit cost < 1
    with pytest.raises(lrl.LRError):
        gac.select([1.0], [1], [5.0], [[]], 100)        # no candidate
    with pytest.raises(lrl.LRError):
        gac.select([1.0], [1], [5.0], [[8]], -1)        # negative budget
    with pytest.raises(lrl.LRError) as e:
        gac.select([1.0] * 4, [1] * 4, [5.0] * 4, [[8]] * 4, 1 << 40, 1)  # table too large
    assert e.value.status == lrl.LR_ERR_UNSUPPORTED
    del ctypes
