"""GPU test of lr_decode_noalloc, the entry point that allocates nothing:
its output against lr_linear_run's on a handle made with the default flags
(the same kernel and plan), and against the oracle, on two calls in a row
with the second smaller than the first."""
import ctypes

import numpy as np
import pytest

import oracle
import rank_linear_layer_amd as lrl
from rank_linear_layer_amd import datagen
from tests.gpu_util import assert_parity, banner, to_bits, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def gpu():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    lrl.load_library()
    return torch


def _noalloc(torch, X, A, B, status):
    M, N = X.shape[0], B.shape[1]
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device="cuda")
    return lrl.decode_noalloc(X, A, B, Y, status=status)


@pytest.mark.parametrize("cases", [
    ((8, 4096, 1637, 4096), (3, 1024, 300, 1000)),      # q_proj, then a smaller ragged shape
    ((16, 4096, 2867, 14336), (1, 14336, 2867, 4096)),  # gate/up at the largest M, then down at M = 1
])
def test_noalloc_matches_handle_path(gpu, cases):
    torch = gpu
    status = torch.zeros(1, dtype=torch.int32, device="cuda")
    for i, (M, K, r, N) in enumerate(cases):
        banner("noalloc call %d: M=%d K=%d r=%d N=%d" % (i, M, K, r, N))
        Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 9100 + 7 * i + r)
        X, A, B = to_dev(Xb), to_dev(Ab), to_dev(Bb)
        y_free = to_bits(_noalloc(torch, X, A, B, status))
        lin = lrl.LowRankLinear(A, B, max_M=M, flags=lrl.LR_FLAG_FACTORED)
        y_handle = to_bits(lin(X))
        assert np.array_equal(y_free, y_handle), "call %d differs from lr_linear_run" % i
        assert_parity(y_free, oracle.lowrank_bf16(Xb, Ab, Bb), "noalloc call %d" % i)
        del lin
    torch.cuda.synchronize()
    assert int(status.item()) == 0


def test_noalloc_repeated_and_graph_captured(gpu):
    # the scratch array keeps the last call's contents: alternating shapes,
    # eager and replayed from a graph, every result equal to the first
    torch = gpu
    shapes = [(8, 2048, 777, 2000), (2, 512, 61, 333)]
    data = []
    for j, (M, K, r, N) in enumerate(shapes):
        Xb, Ab, Bb = datagen.factorized_inputs(M, K, r, N, 9300 + j)
        X, A, B = to_dev(Xb), to_dev(Ab), to_dev(Bb)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device="cuda")
        data.append((X, A, B, Y, oracle.lowrank_bf16(Xb, Ab, Bb)))

    def step():
        for X, A, B, Y, _ in data:
            lrl.decode_noalloc(X, A, B, Y)

    step()
    torch.cuda.synchronize()
    first = [to_bits(d[3]).copy() for d in data]
    for j, d in enumerate(data):
        assert_parity(first[j], d[4], "shape %d" % j)
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step()
    for rep in range(3):
        for d in data:
            d[3].fill_(0)
        step()
        torch.cuda.synchronize()
        assert all(np.array_equal(to_bits(d[3]), f) for d, f in zip(data, first)), "eager %d" % rep
        for d in data:
            d[3].fill_(0)
        g.replay()
        torch.cuda.synchronize()
        assert all(np.array_equal(to_bits(d[3]), f) for d, f in zip(data, first)), "replay %d" % rep
    del g


def test_noalloc_rejects_through_the_abi(gpu):
    torch = gpu
    lib = lrl.load_library()
    X = torch.zeros((17, 64), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((64, 8), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((8, 32), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((17, 32), dtype=torch.bfloat16, device="cuda")
    vp = ctypes.c_void_p
    st = lib.lr_decode_noalloc(vp(X.data_ptr()), vp(A.data_ptr()), vp(B.data_ptr()), vp(Y.data_ptr()), 17, 64, 8, 32,
                               None, None)
    assert st == lrl.LR_ERR_INVALID_ARG
    st = lib.lr_decode_noalloc(vp(X.data_ptr()), vp(A.data_ptr()), vp(B.data_ptr()), vp(X.data_ptr()), 4, 64, 8, 32,
                               None, None)
    assert st == lrl.LR_ERR_INVALID_ARG   # Y overlaps X
    # a shape whose exchange tables exceed the array is refused before any
    # launch (K = 4096, r = 2867, N = 40000 at M = 16 needs about 64 MiB)
    M, K, r, N = 16, 4096, 2867, 40000
    X = torch.zeros((M, K), dtype=torch.bfloat16, device="cuda")
    A = torch.zeros((K, r), dtype=torch.bfloat16, device="cuda")
    B = torch.zeros((r, N), dtype=torch.bfloat16, device="cuda")
    Y = torch.zeros((M, N), dtype=torch.bfloat16, device="cuda")
    st = lib.lr_decode_noalloc(vp(X.data_ptr()), vp(A.data_ptr()), vp(B.data_ptr()), vp(Y.data_ptr()), M, K, r, N,
                               None, None)
    assert st == lrl.LR_ERR_UNSUPPORTED
    assert b"scratch" in lib.lr_last_error()
