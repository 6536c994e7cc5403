"""GPU parity: the HIP path (through the C ABI) against the float64 CPU
oracle on the same seeded inputs.

Bar (bf16 in, fp32 accumulate, bf16 out), per output tensor:
    rel_fro = ||Y_gpu - Y_ref||_F / ||Y_ref||_F <= 5e-3
    max_abs = max|Y_gpu - Y_ref| / max|Y_ref|   <= 2e-2
Full-size workloads compare sampled outputs that the oracle computes one by
one; smaller cases compare every element.
"""
import numpy as np
import pytest

import oracle
import rank_linear_layer_amd as lrl
from rank_linear_layer_amd import configs, datagen
from tests.gpu_util import assert_parity, banner, tile_cover, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrl.load_library()  # raises loudly if the HIP library is missing
    return torch


def run_case(M, K, r, N, seed, flags=0, max_M=None, full=True, rows=None, cols=None, auto=False):
    # the factorized kernels unless a case asks for the dense fallback or
    # for the library's own choice (auto)
    if not auto and not flags & lrl.LR_FLAG_DENSE:
        flags |= lrl.LR_FLAG_FACTORED
    banner("case M=%d K=%d r=%d N=%d flags=%d seed=%d" % (M, K, r, N, flags, seed))
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, seed)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=max_M or M, flags=flags)
    Y = lin(to_dev(Xb))
    yb = to_bits(Y)
    if full:
        ref = oracle.lowrank_bf16(Xb, Ab, Bb)
        p = assert_parity(yb, ref, "M=%d K=%d r=%d N=%d" % (M, K, r, N))
    else:
        ref = oracle.lowrank_bf16_sampled(Xb, Ab, Bb, rows, cols)
        p = assert_parity(yb[np.ix_(rows, cols)], ref, "sampled M=%d K=%d r=%d N=%d" % (M, K, r, N))
        assert np.all(np.isfinite(datagen.bf16_bits_to_f32(yb))), "non-finite output"
    return p, lin, (Xb, Ab, Bb), yb


# ------------------------------------------------------------ workloads ---

DECODE_KERNELS = [0, lrl.LR_FLAG_DECODE_STREAMING, lrl.LR_FLAG_DECODE_RESIDENT, lrl.LR_FLAG_DECODE_XCD]


@pytest.mark.parametrize("M", [1, 8, 16])
@pytest.mark.parametrize("dflag", DECODE_KERNELS)
def test_tiny_decode(M, dflag):
    c = configs.TINY
    run_case(M, c["K"], c["r"], c["N"], configs.seed_base(0), flags=dflag)


@pytest.mark.parametrize("M", [16, 17, 200])
def test_tiny_prefill(M):
    c = configs.TINY
    run_case(M, c["K"], c["r"], c["N"], configs.seed_base(0) + 3, flags=lrl.LR_FLAG_FORCE_PREFILL)


def test_eckart_young_factors_decode_and_prefill(gpu):
    torch = gpu
    c = configs.EY
    W, A64, B64, Ab, Bb = datagen.svd_factor_inputs(c["K"], c["N"], c["k"], c["w_seed"])
    # X random (decode) and X = I (prefill, Y = the rank-5 reconstruction)
    Xb = datagen.normal_bf16((16, c["K"]), 1.0, c["x_seed"])
    eye = datagen.bf16_bits_from_f32(np.eye(c["K"], dtype=np.float32))
    for X_bits, flags in ((Xb, 0), (eye, 0), (eye[:16], lrl.LR_FLAG_FORCE_DECODE)):
        M = X_bits.shape[0]
        banner("eckart-young M=%d flags=%d" % (M, flags))
        lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags)
        yb = to_bits(lin(to_dev(X_bits)))
        ref = oracle.lowrank_bf16(X_bits, Ab, Bb)
        assert_parity(yb, ref, "EY M=%d" % M)
    # X = I: the GPU reconstruction error is the tail energy of W's spectrum
    # up to the bf16 rounding of factors and output.
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=c["K"])
    Y = datagen.bf16_bits_to_f32(to_bits(lin(to_dev(eye)))).astype(np.float64)
    S = np.linalg.svd(W, compute_uv=False)
    tail = float(np.sum(S[c["k"]:] ** 2))
    assert abs(float(np.sum((W - Y) ** 2)) - tail) <= 2e-3 * tail
    del torch


@pytest.mark.parametrize("dflag", DECODE_KERNELS)
def test_qproj_decode_full(dflag):
    c = configs.QPROJ_DECODE
    p, lin, _, _ = run_case(c["M"], c["K"], c["r"], c["N"], configs.seed_base(c["index"]), flags=dflag)
    banner("q_proj decode parity %s plan %s" % (p, lin.describe()))


# Prefill tiles are 256 rows by 192, 224 or 256 columns (phase 2) and the
# k-split / tile walk differs per plan, so the sampled checks take one row in
# every 256-row block and one column in every 128-column block (every output
# tile holds at least one sampled element), plus tile edges and the ragged end.
def _cover(M, N, seed):
    rows = tile_cover(M, 256, seed, extra=(1, 255, 256, M - 2))
    cols = tile_cover(N, 128, seed + 1, extra=(1, 191, 192, 223, 224, 255, 256, N - 2))
    return rows, cols


def test_mlp_up_prefill_sampled():
    c = configs.MLP_UP_PREFILL
    rows, cols = _cover(c["M"], c["N"], 600)
    p, lin, _, _ = run_case(c["M"], c["K"], c["r"], c["N"], configs.seed_base(c["index"]), full=False,
                            rows=rows, cols=cols)
    banner("mlp_up prefill sampled parity %s plan %s" % (p, lin.describe()))


@pytest.mark.parametrize("name", ["q", "k", "gate", "down"])
def test_layer_projections_decode_m1(name):
    proj = {p.name: p for p in configs.LAYER_PROJS}[name]
    idx = [p.name for p in configs.LAYER_PROJS].index(name)
    run_case(1, proj.K, proj.r, proj.N, configs.seed_base(configs.LAYER_INDEX, idx))


@pytest.mark.parametrize("name", ["q", "k", "v", "o", "gate", "up", "down"])
def test_layer_projections_prefill_m2048_sampled(name):
    # every projection of the bench's layer line at M = 2048 (q, k, o, down
    # have fewer output tiles than compute units, so their plans split k)
    proj = {p.name: p for p in configs.LAYER_PROJS}[name]
    idx = [p.name for p in configs.LAYER_PROJS].index(name)
    rows, cols = _cover(2048, proj.N, 700 + idx)
    p, lin, _, _ = run_case(2048, proj.K, proj.r, proj.N, configs.seed_base(configs.LAYER_INDEX, idx), full=False,
                            rows=rows, cols=cols)
    banner("layer %s M=2048 sampled parity %s plan %s" % (name, p, lin.describe()))


@pytest.mark.parametrize("N,r", [(4096, 1000), (3999, 1001), (3999, 1037), (4096, 1063), (3999, 1100)])
def test_alignment_sweep_points(N, r):
    seed = configs.sweep_seed(N, r)
    run_case(1, configs.SWEEP_K, r, N, seed)
    rows, cols = _cover(512, N, seed)
    run_case(512, configs.SWEEP_K, r, N, seed, full=False, rows=rows, cols=cols)


# ----------------------------------------------------- adversarial grid ---

GRID = []
_r = [1, 2, 5, 7, 8, 15, 16, 17, 31, 32, 33, 119, 120, 121, 240, 241]
_N = [1, 7, 48, 119, 120, 121, 239, 241, 3999]
_M = [1, 2, 5, 15, 16, 17, 31, 64, 130]
_K = [8, 31, 64, 100, 257, 33]
for i, r in enumerate(_r):
    for j in range(3):
        GRID.append((_M[(i + 3 * j) % len(_M)], _K[(i + j) % len(_K)], r, _N[(2 * i + j) % len(_N)]))


@pytest.mark.parametrize("M,K,r,N", GRID)
def test_adversarial_shapes(M, K, r, N):
    run_case(M, K, r, N, 9000 + 31 * r + N + M)


# decode shapes that fit the LDS-resident kernel (K % 8 == 0), both kernels
RES_GRID = [(1, 8, 1, 1), (3, 64, 5, 48), (16, 256, 129, 257), (7, 2048, 255, 300), (2, 512, 128, 128),
            (5, 512, 383, 3999), (16, 8192, 64, 64), (1, 4096, 1100, 3999)]


@pytest.mark.parametrize("M,K,r,N", RES_GRID)
@pytest.mark.parametrize("dflag", DECODE_KERNELS)
def test_decode_kernels_resident_shapes(M, K, r, N, dflag):
    run_case(M, K, r, N, 7100 + r + N + M, flags=dflag)


@pytest.mark.parametrize("M,K,r,N,flags", [(3, 96, 13, 29, lrl.LR_FLAG_FORCE_PREFILL),
                                           (40, 40, 9, 17, 0), (16, 2000, 300, 250, lrl.LR_FLAG_FORCE_PREFILL),
                                           (2, 2000, 300, 250, 0)])
def test_forced_paths(M, K, r, N, flags):
    run_case(M, K, r, N, 4400 + M, flags=flags)


# k-split prefill plans (fp32 partials + reduction kernel), including the
# misaligned-X path (K mod 8 != 0), a ragged M and both tile widths
@pytest.mark.parametrize("M,K,r,N", [(300, 4100, 100, 200), (257, 4096, 131, 999), (600, 2050, 77, 3001),
                                     (33, 8192, 40, 64), (512, 1030, 250, 4100)])
def test_prefill_k_split_plans(M, K, r, N):
    p, lin, _, _ = run_case(M, K, r, N, 5100 + M + r)
    banner("k-split case M=%d K=%d r=%d N=%d parity %s plan %s" % (M, K, r, N, p, lin.describe()))


# A NaN stays where it belongs.  X rows and B rows are loaded from their
# exact first element, so the chunk that ends a row also brings in the next
# row's first elements: for X (K mod 8 != 0) the kernel clears them before
# the MFMAs, and for B (N mod 8 != 0) they only reach output columns past N,
# which are never stored.  NaN rows of X must give NaN rows of Y and nothing
# else; a NaN in B's column 0 must give a NaN column 0 and nothing else.
@pytest.mark.parametrize("flags", [0, lrl.LR_FLAG_PREFILL_TWO_WAVE])
@pytest.mark.parametrize("K", [100, 1001])
def test_nan_stays_in_its_row_and_column(gpu, flags, K):
    M, r, N = 300, 77, 203
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 5300 + K)
    Xb, Bb = Xb.copy(), Bb.copy()
    bad_rows = [1, 17, 255, 256, 299]
    Xb[bad_rows, 0] = 0x7FC0  # bf16 quiet NaN
    Bb[[5, 40], 0] = 0x7FC0
    banner("nan case M=%d K=%d r=%d N=%d flags=%d" % (M, K, r, N, flags))
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags | lrl.LR_FLAG_FACTORED)
    yb = to_bits(lin(to_dev(Xb)))
    y = datagen.bf16_bits_to_f32(yb)
    good = np.setdiff1d(np.arange(M), bad_rows)
    assert np.all(np.isnan(y[bad_rows])), "NaN rows of X must give NaN rows of Y"
    assert np.all(np.isnan(y[:, 0])), "a NaN in B's column 0 must reach Y's column 0"
    assert np.all(np.isfinite(y[np.ix_(good, np.arange(1, N))])), "NaN leaked into other rows or columns"
    Bc = Bb.copy()
    Bc[[5, 40], 0] = 0
    ref = oracle.lowrank_bf16(Xb[good], Ab, Bc)
    assert_parity(yb[np.ix_(good, np.arange(1, N))], ref[:, 1:], "finite part")


@pytest.mark.parametrize("M", [300])
def test_mlp_packed_prefill_k_split(M):
    # packed gate/up at a small M: the shared plan splits k for both outputs
    K = 2048
    Xb = datagen.normal_bf16((M, K), 1.0, 61)
    _, Agb, Bgb = datagen.factorized_inputs(1, K, 203, 900, 71)
    _, Aub, Bub = datagen.factorized_inputs(1, K, 150, 1300, 81)
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M)
    Yg, Yu = lrl.mlp_packed(gate, up, to_dev(Xb))
    assert_parity(to_bits(Yg), oracle.lowrank_bf16(Xb, Agb, Bgb), "packed k-split gate")
    assert_parity(to_bits(Yu), oracle.lowrank_bf16(Xb, Aub, Bub), "packed k-split up")


# ------------------------------------------------- prefill kernel kinds ---
# Each prefill kernel forced on its own: the two-wave kernel (256 x 32 nb
# tiles, weight rows read with the transposing LDS read) and the one-wave
# kernel (256 x 256 tiles, weight rows transposed in registers).  Phase 1
# reads A (leading dimension r) and phase 2 reads B (leading dimension N),
# so the first eight shapes cover every r mod 8 and
# N mod 8; the rest add ragged M, partial column tiles, rank padding,
# k-splits and a misaligned X (K mod 8 != 0: phase 1 falls back to the
# two-wave kernel).
KIND_SHAPES = [(300, 512, 256 + q, 512 + (3 * q) % 8) for q in range(8)] + [
    (513, 1024, 645, 2056), (257, 2048, 817, 1024), (40, 4096, 333, 999), (1000, 520, 77, 300),
    (333, 1001, 100, 300)]


def _plan_kinds(lin):
    """(phase-1 kind, phase-2 kind) of the last prefill call, from describe()."""
    import re
    m = re.search(r"phase1 kind=(-?\d+) nb=\d+ splits=\d+, phase2 kind=(-?\d+)", lin.describe())
    return int(m.group(1)), int(m.group(2))


@pytest.mark.parametrize("flags", [lrl.LR_FLAG_PREFILL_TWO_WAVE, lrl.LR_FLAG_PREFILL_ONE_WAVE])
@pytest.mark.parametrize("M,K,r,N", KIND_SHAPES)
def test_prefill_kernel_kinds(M, K, r, N, flags):
    p, lin, _, _ = run_case(M, K, r, N, 6100 + M + r + N, flags=flags)
    k1, k2 = _plan_kinds(lin)
    banner("kinds M=%d K=%d r=%d N=%d flags=%d: phase kinds %d %d parity %s" % (M, K, r, N, flags, k1, k2, p))
    if flags == lrl.LR_FLAG_PREFILL_TWO_WAVE:
        assert (k1, k2) == (0, 0)
    else:
        assert k1 == (1 if K % 8 == 0 else 0) and k2 == 1


def test_mlp_packed_one_wave():
    # packed gate/up through the one-wave kernel (both factors r = 203)
    M, K = 300, 1024
    Xb = datagen.normal_bf16((M, K), 1.0, 63)
    _, Agb, Bgb = datagen.factorized_inputs(1, K, 203, 900, 73)
    _, Aub, Bub = datagen.factorized_inputs(1, K, 203, 1300, 83)
    f = lrl.LR_FLAG_PREFILL_ONE_WAVE
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M, flags=f)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M, flags=f)
    Yg, Yu = lrl.mlp_packed(gate, up, to_dev(Xb))
    assert _plan_kinds(gate) == (1, 1)
    assert_parity(to_bits(Yg), oracle.lowrank_bf16(Xb, Agb, Bgb), "packed one-wave gate")
    assert_parity(to_bits(Yu), oracle.lowrank_bf16(Xb, Aub, Bub), "packed one-wave up")


# ----------------------------------------------------------------- group ---
# n projections sharing X in shared launches (lr_group_run): the q, k and v
# projections of the decoder layer, and smaller groups that reach the
# per-residue launch split, the mixed decode/prefill split and the limits.

def _layer_group(names, M):
    projs = {p.name: (i, p) for i, p in enumerate(configs.LAYER_PROJS)}
    Xb = datagen.normal_bf16((M, 4096), 1.0, configs.seed_base(configs.LAYER_INDEX))
    fac = []
    for nm in names:
        i, p = projs[nm]
        _, Ab, Bb = datagen.factorized_inputs(1, p.K, p.r, p.N, configs.seed_base(configs.LAYER_INDEX, i))
        fac.append((Ab, Bb))
    return Xb, fac


@pytest.mark.parametrize("M", [1, 8, 64, 300])
def test_group_qkv_matches_oracle(M):
    banner("group qkv M=%d" % M)
    Xb, fac = _layer_group(["q", "k", "v"], M)
    lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M) for A, B in fac]
    X = to_dev(Xb)
    Ys = lrl.group_run(lins, X)
    ys = [to_bits(Y) for Y in Ys]
    for nm, y, (A, B) in zip("qkv", ys, fac):
        assert_parity(y, oracle.lowrank_bf16(Xb, A, B), "group %s M=%d" % (nm, M))
    # a repeated group call is bitwise equal; separate runs agree to the bar
    Ys2 = lrl.group_run(lins, X)
    assert all(np.array_equal(y, to_bits(Y2)) for y, Y2 in zip(ys, Ys2))
    for nm, y, lin in zip("qkv", ys, lins):
        assert_parity(y, datagen.bf16_bits_to_f32(to_bits(lin(X))).astype(np.float64), "group vs separate " + nm)
    if M > lrl.LR_DECODE_MAX_M:
        banner("group qkv M=%d plans: %s" % (M, " | ".join(lin.describe().split("xcd_local")[1] for lin in lins)))


def test_group_qkv_m2048_sampled():
    M = 2048
    Xb, fac = _layer_group(["q", "k", "v"], M)
    lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M) for A, B in fac]
    Ys = lrl.group_run(lins, to_dev(Xb))
    for i, (nm, Y, (A, B), lin) in enumerate(zip("qkv", Ys, fac, lins)):
        rows, cols = _cover(M, B.shape[1], 800 + i)
        y = to_bits(Y)
        p = assert_parity(y[np.ix_(rows, cols)], oracle.lowrank_bf16_sampled(Xb, A, B, rows, cols),
                          "group %s M=2048 sampled" % nm)
        assert np.all(np.isfinite(datagen.bf16_bits_to_f32(y)))
        banner("group %s M=2048 sampled parity %s plan %s" % (nm, p, lin.describe()))


# four projections whose A leading dimensions (r) differ mod 8 while the B
# leading dimensions (N) agree: phase 1 runs as one two-wave launch or one
# one-wave launch per residue class, phase 2 as one launch
GROUP4 = [(203, 900), (150, 1300), (99, 517), (211, 260)]


@pytest.mark.parametrize("flags", [0, lrl.LR_FLAG_PREFILL_TWO_WAVE, lrl.LR_FLAG_PREFILL_ONE_WAVE])
@pytest.mark.parametrize("M", [40, 300])
def test_group_four_projections_mixed_residues(M, flags):
    K = 1024
    banner("group4 M=%d flags=%d" % (M, flags))
    Xb = datagen.normal_bf16((M, K), 1.0, 91)
    fac = [datagen.factorized_inputs(1, K, r, N, 101 + 10 * i)[1:] for i, (r, N) in enumerate(GROUP4)]
    # (211, 260) would take the dense fallback by itself: kept factorized here
    f = flags | lrl.LR_FLAG_FACTORED
    lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M, flags=f) for A, B in fac]
    Ys = lrl.group_run(lins, to_dev(Xb))
    for i, (Y, (A, B)) in enumerate(zip(Ys, fac)):
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, A, B), "group4 output %d M=%d flags=%d" % (i, M, flags))
    kinds = [_plan_kinds(lin) for lin in lins]
    banner("group4 M=%d flags=%d kinds %s" % (M, flags, kinds))
    if flags == lrl.LR_FLAG_PREFILL_TWO_WAVE:
        assert all(k == (0, 0) for k in kinds)
    if flags == lrl.LR_FLAG_PREFILL_ONE_WAVE:
        assert all(k == (1, 1) for k in kinds)


def test_group_mixed_decode_and_prefill():
    # at M = 4 a FORCE_PREFILL handle takes the prefill kernels while the
    # others share a decode launch
    M, K = 4, 512
    Xb = datagen.normal_bf16((M, K), 1.0, 93)
    shapes = [(67, 700, 0), (97, 600, lrl.LR_FLAG_FORCE_PREFILL), (33, 128, 0)]
    fac = [datagen.factorized_inputs(1, K, r, N, 201 + 10 * i)[1:] for i, (r, N, _) in enumerate(shapes)]
    lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M, flags=f) for (A, B), (_, _, f) in zip(fac, shapes)]
    Ys = lrl.group_run(lins, to_dev(Xb))
    for i, (Y, (A, B)) in enumerate(zip(Ys, fac)):
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, A, B), "mixed group output %d" % i)
    assert _plan_kinds(lins[1])[0] >= 0


def test_group_errors_on_device():
    K = 256
    fac = [datagen.factorized_inputs(1, K, 17, 64, 301 + i)[1:] for i in range(2)]
    a, b = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=8) for A, B in fac]
    _, A2, B2 = datagen.factorized_inputs(1, 128, 17, 64, 311)
    c = lrl.LowRankLinear(to_dev(A2), to_dev(B2), max_M=8)
    X = to_dev(datagen.normal_bf16((4, K), 1.0, 5))
    with pytest.raises(lrl.LRError) as e:
        lrl.group_run([a, a], X)
    assert e.value.status == lrl.LR_ERR_INVALID_ARG and "same" in str(e.value)
    with pytest.raises(lrl.LRError) as e:
        lrl.group_run([a, c], X)
    assert e.value.status == lrl.LR_ERR_INVALID_ARG and "K=" in str(e.value)
    with pytest.raises(lrl.LRError) as e:
        lrl.group_run([a, b], to_dev(datagen.normal_bf16((9, K), 1.0, 5)))  # M above max_M
    assert e.value.status == lrl.LR_ERR_INVALID_ARG
    Ya, Yb = lrl.group_run([a, b], X)
    with pytest.raises(lrl.LRError):  # outputs overlap
        lrl.group_run([a, b], X, outs=[Ya, Ya])


# ---------------------------------------------------------------- packed ---

@pytest.mark.parametrize("M", [1, 4, 64])
def test_mlp_packed_matches_oracle_and_separate_runs(M):  # noqa: C901
    K, r, N = 512, 67, 700
    banner("packed M=%d" % M)
    Xb = datagen.normal_bf16((M, K), 1.0, 31)
    _, Agb, Bgb = datagen.factorized_inputs(1, K, r, N, 41)
    _, Aub, Bub = datagen.factorized_inputs(1, K, r + 30, N - 100, 51)
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M)
    X = to_dev(Xb)
    Yg, Yu = lrl.mlp_packed(gate, up, X)
    yg, yu = to_bits(Yg), to_bits(Yu)
    assert_parity(yg, oracle.lowrank_bf16(Xb, Agb, Bgb), "packed gate")
    assert_parity(yu, oracle.lowrank_bf16(Xb, Aub, Bub), "packed up")
    # a separate run may plan a different k-split (its own tile count), so
    # it is compared within the bar; a repeated packed run is bitwise equal
    assert_parity(yg, datagen.bf16_bits_to_f32(to_bits(gate(X))).astype(np.float64), "packed vs separate gate")
    assert_parity(yu, datagen.bf16_bits_to_f32(to_bits(up(X))).astype(np.float64), "packed vs separate up")
    Yg2, Yu2 = lrl.mlp_packed(gate, up, X)
    assert np.array_equal(yg, to_bits(Yg2)) and np.array_equal(yu, to_bits(Yu2))


# The last element of A and of B, made large: a kernel that loses it (an
# unaligned load that reaches past a matrix ending on a dword boundary reads
# it as zero) misses the bar by far.  Shapes with K*r and r*N even and odd.
LAST_SHAPES = [(300, 512, 259, 514), (64, 256, 258, 1001), (40, 1024, 97, 66), (33, 96, 255, 257)]


@pytest.mark.parametrize("flags", [lrl.LR_FLAG_PREFILL_ONE_WAVE, lrl.LR_FLAG_PREFILL_TWO_WAVE, 0] + DECODE_KERNELS[1:])
@pytest.mark.parametrize("M,K,r,N", LAST_SHAPES)
def test_last_elements_count(M, K, r, N, flags):
    if flags in DECODE_KERNELS:
        M = min(M, 8)
    banner("last elements M=%d K=%d r=%d N=%d flags=%d" % (M, K, r, N, flags))
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 9500 + r)
    Ab, Bb = Ab.copy(), Bb.copy()
    Ab[-1, -1] = 0x4100  # bf16 8.0
    Bb[-1, -1] = 0x4100
    Xb = Xb.copy()
    Xb[:, -1] = 0x3F80   # bf16 1.0: the last row of A reaches every output row
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags | lrl.LR_FLAG_FACTORED)
    assert_parity(to_bits(lin(to_dev(Xb))), oracle.lowrank_bf16(Xb, Ab, Bb), "last elements flags=%d" % flags)


def _gate_up(M):
    Xb, fac = _layer_group(["gate", "up"], M)
    (Agb, Bgb), (Aub, Bub) = fac
    return Xb, Agb, Bgb, Aub, Bub


def test_mlp_packed_gate_up_m2048_sampled():
    # the bench layer line's packed gate/up at M = 2048 (K 4096, r 2867,
    # N 14336 each), every output tile sampled, against the oracle and
    # against single calls of each handle
    M = 2048
    banner("packed gate/up M=%d" % M)
    Xb, Agb, Bgb, Aub, Bub = _gate_up(M)
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M)
    X = to_dev(Xb)
    Yg, Yu = lrl.mlp_packed(gate, up, X)
    for i, (nm, Y, A, B, lin) in enumerate((("gate", Yg, Agb, Bgb, gate), ("up", Yu, Aub, Bub, up))):
        rows, cols = _cover(M, B.shape[1], 900 + i)
        y = to_bits(Y)
        p = assert_parity(y[np.ix_(rows, cols)], oracle.lowrank_bf16_sampled(Xb, A, B, rows, cols), "packed " + nm)
        assert np.all(np.isfinite(datagen.bf16_bits_to_f32(y)))
        ys = to_bits(lin(X))
        assert_parity(y, datagen.bf16_bits_to_f32(ys).astype(np.float64), "packed vs single " + nm)
        banner("packed %s M=2048 sampled parity %s plan %s" % (nm, p, lin.describe()))


@pytest.mark.parametrize("flags", [0, lrl.LR_FLAG_DECODE_XCD, lrl.LR_FLAG_DECODE_SPLIT])
@pytest.mark.parametrize("M", [1, 8])
def test_mlp_packed_gate_up_layer_decode(flags, M):
    # the bench layer line's packed gate/up at decode, full output against
    # the oracle, for the default kernel and the two opt-in ones
    banner("packed gate/up decode M=%d flags=%d" % (M, flags))
    Xb, Agb, Bgb, Aub, Bub = _gate_up(M)
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M, flags=flags | lrl.LR_FLAG_FACTORED)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M, flags=flags | lrl.LR_FLAG_FACTORED)
    Yg, Yu = lrl.mlp_packed(gate, up, to_dev(Xb))
    assert_parity(to_bits(Yg), oracle.lowrank_bf16(Xb, Agb, Bgb), "packed decode gate")
    assert_parity(to_bits(Yu), oracle.lowrank_bf16(Xb, Aub, Bub), "packed decode up")


def test_packed_half_plans_alternate_with_single_runs(gpu):
    # gate and up (register-streaming decode) do not fit one launch on their
    # own plans, so the packed call runs both on their half-machine plans in
    # the same decode tables; single calls use the full plans.  Alternating
    # the two, eager and from a captured graph, every output must equal the
    # first (stale epoch-tagged words of the other plan must never match).
    torch = gpu
    M = 1
    banner("packed half plans alternating with single runs, M=%d" % M)
    Xb, Agb, Bgb, Aub, Bub = _gate_up(M)
    X = to_dev(Xb)
    gate = lrl.LowRankLinear(to_dev(Agb), to_dev(Bgb), max_M=M)
    up = lrl.LowRankLinear(to_dev(Aub), to_dev(Bub), max_M=M)
    assert "kind=streaming" in gate.describe()
    ref_g, ref_u = oracle.lowrank_bf16(Xb, Agb, Bgb), oracle.lowrank_bf16(Xb, Aub, Bub)
    Yg, Yu = lrl.mlp_packed(gate, up, X)
    first_g, first_u = to_bits(Yg), to_bits(Yu)
    assert_parity(first_g, ref_g, "packed gate")
    assert_parity(first_u, ref_u, "packed up")
    for it in range(3):
        yg1, yu1 = to_bits(gate(X)), to_bits(up(X))
        assert_parity(yg1, ref_g, "single gate, round %d" % it)
        assert_parity(yu1, ref_u, "single up, round %d" % it)
        Yg, Yu = lrl.mlp_packed(gate, up, X)
        assert np.array_equal(to_bits(Yg), first_g) and np.array_equal(to_bits(Yu), first_u), "round %d" % it
    # graph replays of the packed call, with single eager calls between them
    Og = torch.empty_like(Yg)
    Ou = torch.empty_like(Yu)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        lrl.mlp_packed(gate, up, X, Og, Ou)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        lrl.mlp_packed(gate, up, X, Og, Ou)
    for it in range(3):
        Og.zero_()
        Ou.zero_()
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(Og), first_g) and np.array_equal(to_bits(Ou), first_u), "replay %d" % it
        assert_parity(to_bits(gate(X)), ref_g, "single gate after replay %d" % it)
    assert gate.status() == 0 and up.status() == 0


# ----------------------------------------------------------- dense fallback ---
# W = A.B formed at create; decode reads its MFMA-operand layout with no
# exchange between workgroups, prefill runs X.W through the prefill GEMM.
# Cases: the k/v layer shape (auto: its factors hold 99.7% of the dense
# bytes), forced on the q shape, misaligned K (X rows realigned per lane),
# N past a 16-column group, ragged M, tiny shapes.
DENSE_CASES = [(1, 4096, 817, 1024, 0), (8, 4096, 817, 1024, 0), (16, 4096, 817, 1024, 0),
               (8, 4096, 1637, 4096, lrl.LR_FLAG_DENSE), (5, 1001, 700, 300, lrl.LR_FLAG_DENSE),
               (16, 4096, 1063, 3999, lrl.LR_FLAG_DENSE), (1, 8, 3, 1, 0), (3, 33, 40, 17, 0),
               (300, 1024, 645, 1000, lrl.LR_FLAG_DENSE), (40, 520, 400, 300, lrl.LR_FLAG_DENSE),
               (513, 1001, 900, 700, 0), (4, 64, 5, 48, lrl.LR_FLAG_DENSE | lrl.LR_FLAG_FORCE_PREFILL),
               # deep and narrow: decode cuts K into slices whose fp32 partials the last
               # workgroup of each column group adds
               (1, 14336, 2867, 1024, lrl.LR_FLAG_DENSE), (16, 14336, 900, 1000, lrl.LR_FLAG_DENSE),
               (7, 8200, 1000, 40, lrl.LR_FLAG_DENSE)]


def _expect_dense(K, r, N, flags):
    """The library's rule: forced, or the factors hold >= 95% of K x N."""
    if flags & lrl.LR_FLAG_DENSE:
        return True
    return 100 * r * (K + N) >= 95 * K * N


@pytest.mark.parametrize("M,K,r,N,flags", DENSE_CASES)
def test_dense_fallback(M, K, r, N, flags):
    assert _expect_dense(K, r, N, flags)
    p, lin, _, _ = run_case(M, K, r, N, 9100 + M + K + r + N, flags=flags, auto=True)
    assert "dense=1" in lin.describe()
    banner("dense M=%d K=%d r=%d N=%d flags=%d parity %s" % (M, K, r, N, flags, p))


def test_dense_fallback_m2048_sampled():
    # the k/v projection at M = 2048: one GEMM X.W instead of two
    proj = {p.name: p for p in configs.LAYER_PROJS}["k"]
    rows = np.array([0, 1, 255, 256, 1500, 2047])
    cols = np.unique(np.concatenate([np.arange(0, 9), np.arange(500, 520), np.arange(proj.N - 9, proj.N)]))
    p, lin, _, _ = run_case(2048, proj.K, proj.r, proj.N, 9300, flags=lrl.LR_FLAG_DENSE, full=False,
                            rows=rows, cols=cols)
    assert "dense=1" in lin.describe()
    banner("dense k M=2048 sampled parity %s plan %s" % (p, lin.describe()))


def test_dense_choice_follows_the_rule():
    K = 512
    for r, N, flags in [(107, 512, 0), (250, 512, 0), (240, 512, 0), (250, 512, lrl.LR_FLAG_FACTORED),
                        (20, 512, lrl.LR_FLAG_DENSE)]:
        _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 17)
        lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=4, flags=flags)
        want = _expect_dense(K, r, N, flags) and not flags & lrl.LR_FLAG_FACTORED
        assert ("dense=1" in lin.describe()) == want, (r, N, flags, lin.describe())


def test_group_mixed_dense_and_factored():
    # q factorized, k and v dense (auto) in one group: decode and prefill
    for M in (4, 300):
        Xb, fac = _layer_group(["q", "k", "v"], M)
        lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M) for A, B in fac]
        assert [("dense=1" in lin.describe()) for lin in lins] == [False, True, True]
        Ys = lrl.group_run(lins, to_dev(Xb))
        for nm, Y, (A, B) in zip("qkv", Ys, fac):
            assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, A, B), "mixed group %s M=%d" % (nm, M))


@pytest.mark.parametrize("M,K", [(1, 1001), (7, 512), (16, 2048)])
def test_group_dense_projections_one_launch(M, K):
    # several dense-fallback projections sharing X run as one launch; each
    # output equals its own call bitwise and meets the oracle
    shapes = [(K, 40, 1000), (K, 8, 33), (K, 64, 4097), (K, 16, 17)]
    fac = [datagen.factorized_inputs(1, k, r, n, 8100 + i)[1:] for i, (k, r, n) in enumerate(shapes)]
    Xb = datagen.normal_bf16((M, K), 1.0, 8199)
    X = to_dev(Xb)
    lins = [lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M, flags=lrl.LR_FLAG_DENSE) for A, B in fac]
    Ys = lrl.group_run(lins, X)
    for i, (lin, Y, (A, B)) in enumerate(zip(lins, Ys, fac)):
        yb = to_bits(Y)
        assert np.array_equal(yb, to_bits(lin(X))), "grouped dense output %d differs from its own call" % i
        assert_parity(yb, oracle.lowrank_bf16(Xb, A, B), "grouped dense %d M=%d K=%d" % (i, M, K))


# ----------------------------------------------------- invariants/edges ---

@pytest.mark.parametrize("M,N,flags", [(3, 3999, 0), (33, 3999, 0), (5, 241, lrl.LR_FLAG_FORCE_PREFILL),
                                       (3, 241, lrl.LR_FLAG_DENSE), (33, 3999, lrl.LR_FLAG_DENSE)])
def test_canary_guards_and_poison(gpu, M, N, flags):
    torch = gpu
    K, r = 256, 37
    if not flags & lrl.LR_FLAG_DENSE:
        flags |= lrl.LR_FLAG_FACTORED
    banner("canary M=%d N=%d flags=%d" % (M, N, flags))
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 77)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags)
    G = 64  # guard elements on each side (128 bytes keeps Y 16-byte aligned)
    poison = 0x7FC1
    big = torch.full((M * N + 2 * G,), poison, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    Y = big[G:G + M * N].view(M, N)
    lin(to_dev(Xb), out=Y)
    allbits = to_bits(big)
    assert np.all(allbits[:G] == poison) and np.all(allbits[G + M * N:] == poison), "guard zone written"
    assert_parity(allbits[G:G + M * N].reshape(M, N), oracle.lowrank_bf16(Xb, Ab, Bb), "canary")


@pytest.mark.parametrize("M,flags", [(8, 0), (8, lrl.LR_FLAG_DECODE_STREAMING), (8, lrl.LR_FLAG_DECODE_RESIDENT),
                                     (8, lrl.LR_FLAG_DECODE_XCD), (8, lrl.LR_FLAG_DECODE_SPLIT),
                                     (8, lrl.LR_FLAG_DENSE), (48, 0)])
@pytest.mark.parametrize("K", [1024, 14336])
def test_deterministic_bitwise(M, flags, K):
    r, N = 333, 1500
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 1234)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags)
    X = to_dev(Xb)
    outs = [to_bits(lin(X)) for _ in range(3)]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[1], outs[2])


def test_repeated_calls_new_inputs_and_streams(gpu):
    torch = gpu
    K, r, N = 700, 150, 900
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 555)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=16)
    side = torch.cuda.Stream()
    for i, M in enumerate([1, 16, 7, 16, 3, 1]):
        Xb = datagen.normal_bf16((M, K), 1.0, 600 + i)
        X = to_dev(Xb)
        if i % 2:
            with torch.cuda.stream(side):
                Y = lin(X)
            side.synchronize()
        else:
            Y = lin(X)
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "call %d M=%d" % (i, M))


# role-split decode kernel: shapes whose plan fits it (K of any residue)
SPLIT_GRID = [(1, 8, 1, 1), (16, 33, 5, 7), (5, 100, 17, 121), (3, 257, 241, 3999), (8, 4096, 1637, 4096),
              (16, 4100, 1000, 4096), (2, 2000, 300, 250), (7, 4096, 2048, 2048), (1, 4096, 1100, 3999),
              (16, 1, 1, 1), (3, 7, 33, 16), (9, 3, 2, 5000)]


@pytest.mark.parametrize("M,K,r,N", SPLIT_GRID)
def test_split_decode_shapes(M, K, r, N):
    p, lin, _, _ = run_case(M, K, r, N, 7300 + r + N + M, flags=lrl.LR_FLAG_DECODE_SPLIT)
    assert "kind=split" in lin.describe(), lin.describe()


# streaming-Y role-split kernel: B too large for the Y producers' registers
SPLIT_STREAM_GRID = [(1, 4096, 2867, 14336, 1), (8, 4096, 2867, 14336, 8), (4, 2048, 2867, 9000, 4),
                     (3, 1001, 2500, 9001, 3), (12, 2048, 2000, 12000, 12), (9, 2048, 2000, 12000, 16),
                     (1, 512, 4096, 64, 1), (2, 300, 1500, 20000, 2), (1, 2, 4096, 8, 1)]


@pytest.mark.parametrize("M,K,r,N,max_M", SPLIT_STREAM_GRID)
def test_split_stream_decode_shapes(M, K, r, N, max_M):
    p, lin, _, _ = run_case(M, K, r, N, 7700 + r + N + M, max_M=max_M, flags=lrl.LR_FLAG_DECODE_SPLIT)
    assert "kind=split_stream" in lin.describe(), lin.describe()


def test_split_stream_repeated_calls(gpu):
    # one handle, M changing within max_M = 8, several streams, then many
    # launches back to back
    torch = gpu
    K, r, N = 1500, 2100, 9000
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 557)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=8, flags=lrl.LR_FLAG_FACTORED | lrl.LR_FLAG_DECODE_SPLIT)
    assert "kind=split_stream" in lin.describe(), lin.describe()
    side = torch.cuda.Stream()
    for i, M in enumerate([1, 8, 5, 8, 2, 1]):
        Xb = datagen.normal_bf16((M, K), 1.0, 720 + i)
        X = to_dev(Xb)
        if i % 2:
            with torch.cuda.stream(side):
                Y = lin(X)
            side.synchronize()
        else:
            Y = lin(X)
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split_stream call %d M=%d" % (i, M))
    Xb = datagen.normal_bf16((3, K), 1.0, 798)
    X = to_dev(Xb)
    for _ in range(100):
        Y = lin(X)
    torch.cuda.synchronize()
    assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split_stream after 100 launches")


# flat role-split kernel: A-heavy shapes (every workgroup takes a share of A)
SPLIT_FLAT_GRID = [(1, 14336, 2867, 4096, 1), (4, 14336, 2867, 4096, 4), (2, 12001, 2000, 6000, 2),
                   (12, 12000, 1800, 9000, 12), (7, 12000, 1800, 9000, 8)]


@pytest.mark.parametrize("M,K,r,N,max_M", SPLIT_FLAT_GRID)
def test_split_flat_decode_shapes(M, K, r, N, max_M):
    p, lin, _, _ = run_case(M, K, r, N, 7900 + r + N + M, max_M=max_M, flags=lrl.LR_FLAG_DECODE_SPLIT)
    assert "kind=split_flat" in lin.describe(), lin.describe()


def test_split_flat_repeated_calls(gpu):
    torch = gpu
    K, r, N = 12001, 2000, 6000
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 558)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=8, flags=lrl.LR_FLAG_FACTORED | lrl.LR_FLAG_DECODE_SPLIT)
    assert "kind=split_flat" in lin.describe(), lin.describe()
    side = torch.cuda.Stream()
    for i, M in enumerate([1, 8, 3, 8, 1]):
        Xb = datagen.normal_bf16((M, K), 1.0, 740 + i)
        X = to_dev(Xb)
        if i % 2:
            with torch.cuda.stream(side):
                Y = lin(X)
            side.synchronize()
        else:
            Y = lin(X)
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split_flat call %d M=%d" % (i, M))
    Xb = datagen.normal_bf16((2, K), 1.0, 797)
    X = to_dev(Xb)
    for _ in range(100):
        Y = lin(X)
    torch.cuda.synchronize()
    assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split_flat after 100 launches")


def test_split_decode_repeated_calls(gpu):
    # the generation word advances once per launch: many calls on one
    # handle, M changing, on two streams, each against the oracle
    torch = gpu
    K, r, N = 1000, 333, 1500
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 556)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=16, flags=lrl.LR_FLAG_DECODE_SPLIT | lrl.LR_FLAG_FACTORED)
    assert "kind=split" in lin.describe()
    side = torch.cuda.Stream()
    for i, M in enumerate([1, 16, 7, 16, 3, 1, 9, 16]):
        Xb = datagen.normal_bf16((M, K), 1.0, 700 + i)
        X = to_dev(Xb)
        if i % 2:
            with torch.cuda.stream(side):
                Y = lin(X)
            side.synchronize()
        else:
            Y = lin(X)
        assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split call %d M=%d" % (i, M))
    # many launches back to back, then one checked
    Xb = datagen.normal_bf16((4, K), 1.0, 799)
    X = to_dev(Xb)
    for _ in range(200):
        Y = lin(X)
    torch.cuda.synchronize()
    assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, Ab, Bb), "split after 200 launches")


@pytest.mark.parametrize("flags,width", [(lrl.LR_FLAG_DECODE_STREAMING, 120), (0, 32)])
def test_zero_rank_padding_gpu(gpu, flags, width):
    # zero columns of A and rows of B leave the result bitwise unchanged
    # while the kernel's partition of the rank does not change (120-column
    # slices for the streaming kernel, 32-deep k-steps for the role-split
    # one); otherwise the result still meets the oracle
    torch = gpu
    M, K, r, N = 8, 512, 107, 512
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 808)
    X = to_dev(Xb)
    base = to_bits(lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=flags)(X))
    for p in (1, 13, 21, 200):
        Ap = np.concatenate([Ab, np.zeros((K, p), np.uint16)], axis=1)
        Bp = np.concatenate([Bb, np.zeros((p, N), np.uint16)], axis=0)
        yp = to_bits(lrl.LowRankLinear(to_dev(Ap), to_dev(Bp), max_M=M, flags=flags)(X))
        if (r + p + width - 1) // width == (r + width - 1) // width:
            assert np.array_equal(yp, base), "padding by %d changed the result" % p
        else:
            assert_parity(yp, oracle.lowrank_bf16(Xb, Ab, Bb), "padded by %d" % p)
    del torch


def test_error_paths_on_device(gpu):
    torch = gpu
    K, r, N = 64, 5, 48
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 3)
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=4)
    X = to_dev(datagen.normal_bf16((5, K), 1.0, 4))
    with pytest.raises(lrl.LRError) as ei:
        lin(X)  # M = 5 > max_M
    assert ei.value.status == lrl.LR_ERR_INVALID_ARG
    # M = 0 launches nothing and succeeds
    Y0 = lin(X[:0])
    assert Y0.shape == (0, N)
    # Y overlapping X is rejected
    buf = torch.zeros(4 * max(K, N) + 64, dtype=torch.bfloat16, device="cuda")
    Xv = buf[:4 * K].view(4, K)
    Yv = buf[:4 * N].view(4, N)
    import ctypes
    st = lrl.load_library().lr_linear_run(lin.handle, ctypes.c_void_p(Xv.data_ptr()), ctypes.c_void_p(Yv.data_ptr()),
                                          4, None)
    assert st == lrl.LR_ERR_INVALID_ARG
    # gate and up with different K are rejected
    _, A2, B2 = datagen.factorized_inputs(1, K + 8, r, N, 5)
    other = lrl.LowRankLinear(to_dev(A2), to_dev(B2), max_M=4)
    with pytest.raises(lrl.LRError):
        lrl.mlp_packed(lin, other, X[:2])


# ------------------------------------------------------------- graph replay ---
# A whole layer (q, k, v grouped; o; gate/up packed; down) captured once in a
# HIP graph and replayed: no launch argument changes between replays (the
# decode kernels stamp their exchanges with a device-side generation).  Each
# replay follows eager work on the same handles and new contents of the
# captured input, and must equal the eager result for those contents.

@pytest.mark.parametrize("M,flags", [(1, 0), (5, lrl.LR_FLAG_DECODE_STREAMING), (3, lrl.LR_FLAG_DECODE_RESIDENT),
                                     (12, lrl.LR_FLAG_DECODE_SPLIT), (64, 0)])
def test_layer_graph_replay(gpu, M, flags):
    torch = gpu
    banner("graph replay M=%d flags=%d" % (M, flags))
    scale = 4  # a quarter-width layer keeps the test short
    projs = [(p.name, p.K // scale, p.r // scale, p.N // scale) for p in configs.LAYER_PROJS]
    lins, fac = {}, {}
    for i, (nm, K, r, N) in enumerate(projs):
        _, A, B = datagen.factorized_inputs(1, K, r, N, 7000 + 10 * i)
        fac[nm] = (A, B)
        lins[nm] = lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M, flags=flags)
    K0, H = projs[0][1], projs[-1][1]
    X = torch.empty((M, K0), dtype=torch.bfloat16, device="cuda")
    Hin = torch.empty((M, H), dtype=torch.bfloat16, device="cuda")
    outs = {nm: torch.empty((M, N), dtype=torch.bfloat16, device="cuda") for nm, _, _, N in projs}

    def step():
        lrl.group_run([lins["q"], lins["k"], lins["v"]], X, outs=[outs["q"], outs["k"], outs["v"]])
        lins["o"](X, out=outs["o"])
        lrl.mlp_packed(lins["gate"], lins["up"], X, out_gate=outs["gate"], out_up=outs["up"])
        lins["down"](Hin, out=outs["down"])

    def load_inputs(seed):
        X.copy_(torch.from_numpy(datagen.normal_bf16((M, K0), 1.0, seed).view(np.int16)).view(torch.bfloat16))
        Hin.copy_(torch.from_numpy(datagen.normal_bf16((M, H), 1.0, seed + 1).view(np.int16)).view(torch.bfloat16))

    def snapshot():
        torch.cuda.synchronize()
        return {nm: to_bits(t).copy() for nm, t in outs.items()}

    load_inputs(11)
    step()
    step()  # warm: kernel attributes set outside capture
    eager11 = snapshot()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep, seed in enumerate([11, 23, 11, 37]):
        load_inputs(seed)
        step()  # eager work on the same handles between replays
        ref = snapshot()
        if seed == 11:
            assert all(np.array_equal(ref[nm], eager11[nm]) for nm in outs)
        g.replay()
        got = snapshot()
        for nm in outs:
            assert np.array_equal(got[nm], ref[nm]), "replay %d (%s) differs from eager" % (rep, nm)
    # the last replay against the oracle
    Xb = datagen.normal_bf16((M, K0), 1.0, 37)
    Hb = datagen.normal_bf16((M, H), 1.0, 38)
    for nm, K, r, N in projs:
        A, B = fac[nm]
        src = Hb if nm == "down" else Xb
        assert_parity(got[nm], oracle.lowrank_bf16(src, A, B), "graph %s M=%d" % (nm, M))
    del g


@pytest.mark.parametrize("M,K,r,N,kind", [(1, 4096, 2867, 14336, "split_stream"), (3, 14336, 2867, 4096, "split_flat"),
                                          (8, 4096, 1637, 4096, "split"), (8, 4096, 1637, 4096, "xcd"),
                                          (1, 4096, 2867, 14336, "xcd"), (12, 14336, 2867, 4096, "xcd")])
def test_split_variants_graph_replay(gpu, M, K, r, N, kind):
    # each role-split variant captured with two launches on one handle (so
    # the generation word advances twice per replay), replayed with eager
    # launches of the same handle in between; every replay bitwise equal to
    # the eager result, the last one against the oracle
    torch = gpu
    banner("graph replay %s M=%d K=%d r=%d N=%d" % (kind, M, K, r, N))
    _, Ab, Bb = datagen.factorized_inputs(1, K, r, N, 8300 + r)
    extra = lrl.LR_FLAG_DECODE_XCD if kind == "xcd" else lrl.LR_FLAG_DECODE_SPLIT
    lin = lrl.LowRankLinear(to_dev(Ab), to_dev(Bb), max_M=M, flags=lrl.LR_FLAG_FACTORED | extra)
    assert "kind=%s " % kind in lin.describe(), lin.describe()
    X1 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    X2 = torch.empty((M, K), dtype=torch.bfloat16, device="cuda")
    Y1 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    Y2 = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")

    def load(seed):
        X1.copy_(torch.from_numpy(datagen.normal_bf16((M, K), 1.0, seed).view(np.int16)).view(torch.bfloat16))
        X2.copy_(torch.from_numpy(datagen.normal_bf16((M, K), 1.0, seed + 1).view(np.int16)).view(torch.bfloat16))

    def step():
        lin(X1, out=Y1)
        lin(X2, out=Y2)

    load(5)
    step()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep, seed in enumerate([5, 17, 29]):
        load(seed)
        step()
        torch.cuda.synchronize()
        ref = (to_bits(Y1).copy(), to_bits(Y2).copy())
        g.replay()
        torch.cuda.synchronize()
        assert np.array_equal(to_bits(Y1), ref[0]) and np.array_equal(to_bits(Y2), ref[1]), "replay %d" % rep
    assert_parity(to_bits(Y2), oracle.lowrank_bf16(datagen.normal_bf16((M, K), 1.0, 30), Ab, Bb), "graph %s" % kind)
    del g


def test_handle_released_during_capture(gpu):
    # a handle freed while a graph is being captured (a garbage-collected
    # handle of earlier work) must not invalidate that capture
    torch = gpu
    K, r, N, M = 256, 40, 128, 2
    _, A, B = datagen.factorized_inputs(1, K, r, N, 21)
    keep = lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M)
    spare = lrl.LowRankLinear(to_dev(A), to_dev(B), max_M=M)
    Xb = datagen.normal_bf16((M, K), 1.0, 22)
    X = to_dev(Xb)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
    keep(X, out=Y)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        spare.close()
        keep(X, out=Y)
    Y.zero_()
    g.replay()
    torch.cuda.synchronize()
    assert_parity(to_bits(Y), oracle.lowrank_bf16(Xb, A, B), "after a release during capture")


@pytest.mark.parametrize("flag,kinds", [(0, ("resident", "streaming")), (lrl.LR_FLAG_DECODE_STREAMING, ("streaming",)),
                                        (lrl.LR_FLAG_DECODE_SPLIT, ("split", "split_stream", "split_flat")),
                                        (lrl.LR_FLAG_DECODE_XCD, ("xcd",))])
def test_stalled_wait_is_reported(gpu, flag, kinds):
    # LR_FLAG_TEST_STALL makes the T hand-off wait of every decode launch
    # expect a value nobody stores, with a short spin limit: each launch's
    # waits give up, every workgroup still runs to its end, and the handle
    # reports LR_ERR_HIP once, on the next call or through lr_linear_status.
    # A second handle on the same factors, used before and after, is
    # unaffected and stays correct.
    torch = gpu
    M, K, r, N = 4, 1024, 300, 1000
    banner("stall report flags=%d" % flag)
    Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 8800 + flag % 97)
    A, B, X = to_dev(Ab), to_dev(Bb), to_dev(Xb)
    ref = oracle.lowrank_bf16(Xb, Ab, Bb)
    good = lrl.LowRankLinear(A, B, max_M=M, flags=lrl.LR_FLAG_FACTORED | flag)
    bad = lrl.LowRankLinear(A, B, max_M=M, flags=lrl.LR_FLAG_FACTORED | flag | lrl.LR_FLAG_TEST_STALL)
    kind = bad.describe().split("kind=")[1].split()[0]
    assert kind in kinds, bad.describe()
    assert_parity(to_bits(good(X)), ref, "before the stall")
    assert bad.status() == lrl.LR_OK
    bad(X)                      # enqueued; its waits give up on the device
    torch.cuda.synchronize()    # and the launch ends
    assert bad.status() == lrl.LR_ERR_HIP
    assert "gave up waiting" in lrl.load_library().lr_last_error().decode()
    assert bad.status() == lrl.LR_OK   # reported once
    bad(X)
    torch.cuda.synchronize()
    with pytest.raises(lrl.LRError) as ei:
        bad(X)                  # the report comes back from the next call, which launches nothing
    assert ei.value.status == lrl.LR_ERR_HIP
    assert bad.status() == lrl.LR_OK
    for _ in range(2):
        assert_parity(to_bits(good(X)), ref, "after the stall")
    assert good.status() == lrl.LR_OK
