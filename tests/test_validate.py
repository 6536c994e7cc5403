"""CPU tests of the host-side validation and work partition (lr_validate.h),
compiled with g++ into a small test shim -- the same header the HIP
library includes."""
import ctypes
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "rank_linear_layer_amd", "csrc")

SHIM = r"""
#include "lr_validate.h"
extern "C" {
int t_check_create(long long K, long long r, long long N, unsigned long long A, unsigned long long B,
                   long long max_M, unsigned flags) {
  char err[256];
  return lrv::check_create(K, r, N, (const void*)A, (const void*)B, max_M, flags, err, sizeof err);
}
int t_check_run(long long K, long long r, long long N, long long max_M, unsigned long long A, unsigned long long B,
                unsigned long long X, unsigned long long Y, long long M) {
  char err[256];
  lrv::Shape s{K, r, N, max_M, (const void*)A, (const void*)B};
  return lrv::check_run(s, (const void*)X, (const void*)Y, M, err, sizeof err);
}
int t_check_packed(long long Kg, long long Ku, long long r, long long N, unsigned long long Ag, unsigned long long Bg,
                   unsigned long long Au, unsigned long long Bu, unsigned long long X, unsigned long long Yg,
                   unsigned long long Yu, long long M) {
  char err[256];
  lrv::Shape g{Kg, r, N, 64, (const void*)Ag, (const void*)Bg};
  lrv::Shape u{Ku, r, N, 64, (const void*)Au, (const void*)Bu};
  return lrv::check_packed(g, u, (const void*)X, (const void*)Yg, (const void*)Yu, M, err, sizeof err);
}
void t_partition(long long K, long long r, long long N, int budget, int allow_res, int* out) {
  lrv::DecPart p = lrv::decode_partition(K, r, N, budget, allow_res != 0);
  out[0] = p.Jw; out[1] = p.S; out[2] = p.ktps; out[3] = p.ntps;
  out[4] = p.kind; out[5] = p.js_w; out[6] = p.nt_w;
}
}
"""


@pytest.fixture(scope="module")
def shim(tmp_path_factory):
    d = tmp_path_factory.mktemp("shim")
    src = d / "shim.cpp"
    src.write_text(SHIM)
    so = d / "libshim.so"
    subprocess.run(["g++", "-std=c++17", "-O1", "-shared", "-fPIC", "-Wall", "-I", CSRC, str(src), "-o", str(so)],
                   check=True)
    lib = ctypes.CDLL(str(so))
    ll, ull = ctypes.c_longlong, ctypes.c_ulonglong
    lib.t_check_create.argtypes = [ll, ll, ll, ull, ull, ll, ctypes.c_uint]
    lib.t_check_run.argtypes = [ll, ll, ll, ll, ull, ull, ull, ull, ll]
    lib.t_check_packed.argtypes = [ll, ll, ll, ll, ull, ull, ull, ull, ull, ull, ull, ll]
    lib.t_partition.argtypes = [ll, ll, ll, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    return lib


OK, INVALID, UNSUPPORTED = 0, 1, 2
MB = 1 << 20


def test_create_validation(shim):
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 0) == OK
    assert shim.t_check_create(4096, 1637, 4096, 0, 0x2000000, 16, 0) == INVALID
    assert shim.t_check_create(4096, 0, 4096, 0x100000, 0x2000000, 16, 0) == INVALID
    assert shim.t_check_create(4096, 1637, 4096, 0x100008, 0x2000000, 16, 0) == INVALID  # 8B aligned only
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 8) == UNSUPPORTED
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 4) == OK
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 17, 1) == UNSUPPORTED
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 17, 2) == OK
    assert shim.t_check_create(1 << 25, 8, 8, 0x100000, 0x2000000, 1, 0) == INVALID


def test_run_validation_overlap_and_range(shim):
    K, r, N = 64, 5, 48
    A, B = 100 * MB, 101 * MB
    X, Y = 200 * MB, 300 * MB
    assert shim.t_check_run(K, r, N, 16, A, B, X, Y, 8) == OK
    assert shim.t_check_run(K, r, N, 16, A, B, X, Y, 0) == OK       # no-op
    assert shim.t_check_run(K, r, N, 16, A, B, 0, 0, 0) == OK       # M = 0 needs no pointers
    assert shim.t_check_run(K, r, N, 16, A, B, X, Y, 17) == INVALID  # above max_M
    assert shim.t_check_run(K, r, N, 16, A, B, X, Y, -1) == INVALID
    assert shim.t_check_run(K, r, N, 16, A, B, 0, Y, 4) == INVALID
    assert shim.t_check_run(K, r, N, 16, A, B, X, Y + 2, 4) == INVALID  # misaligned Y
    # Y overlapping X (the last byte of X is the first of Y)
    assert shim.t_check_run(K, r, N, 16, A, B, X, X + 4 * K * 2 - 16, 4) == INVALID
    # Y right after X: fine
    assert shim.t_check_run(K, r, N, 16, A, B, X, X + 4 * K * 2, 4) == OK
    # Y inside A or B
    assert shim.t_check_run(K, r, N, 16, A, B, X, A + 16, 1) == INVALID
    assert shim.t_check_run(K, r, N, 16, A, B, X, B, 1) == INVALID


def test_packed_validation(shim):
    Ag, Bg, Au, Bu = 10 * MB, 11 * MB, 12 * MB, 13 * MB
    X, Yg, Yu = 20 * MB, 30 * MB, 40 * MB
    assert shim.t_check_packed(64, 64, 5, 48, Ag, Bg, Au, Bu, X, Yg, Yu, 4) == OK
    assert shim.t_check_packed(64, 32, 5, 48, Ag, Bg, Au, Bu, X, Yg, Yu, 4) == INVALID
    assert shim.t_check_packed(64, 64, 5, 48, Ag, Bg, Au, Bu, X, Yg, Yg + 16, 4) == INVALID
    assert shim.t_check_packed(64, 64, 5, 48, Ag, Bg, Au, Bu, X, Au, Yu, 4) == INVALID


def _part(shim, K, r, N, budget=256, allow_res=True):
    out = (ctypes.c_int * 7)()
    shim.t_partition(K, r, N, budget, 1 if allow_res else 0, out)
    return list(out)


SHAPES = [(4096, 1637, 4096), (512, 107, 512), (64, 5, 48), (4096, 817, 1024), (4096, 2867, 14336),
          (14336, 2867, 4096), (4096, 1000, 3999), (7, 1, 1), (4096, 5000, 4096), (4096, 1100, 3999), (12, 3, 7)]


@pytest.mark.parametrize("K,r,N", SHAPES)
@pytest.mark.parametrize("allow_res", [True, False])
def test_decode_partition_covers_and_fits(shim, K, r, N, allow_res):
    Jw, S, ktps, ntps, kind, js_w, nt_w = _part(shim, K, r, N, allow_res=allow_res)
    assert Jw == -(-r // js_w) or (kind == 1 and Jw * js_w >= r)
    nk, nn = -(-K // 32), -(-N // nt_w)
    assert S * ktps >= nk and S * ntps >= nn   # every tile is owned
    assert (S - 1) * ktps < nk or (S - 1) * ntps < nn  # no fully idle slice
    assert S >= 1 and ktps >= 1 and ntps >= 1
    if kind == 1:
        # resident kernel: one workgroup per CU, slabs fit the LDS plan
        assert allow_res and K % 8 == 0 and nt_w == 128
        assert js_w % 8 == 0 and 8 <= js_w <= 128 and Jw % 8 == 0 and Jw * js_w >= r
        assert Jw * S <= 256 and ktps <= 8 and ntps <= 2
    else:
        assert (js_w, nt_w) == (120, 120)
        assert Jw * S <= max(256, Jw)


def test_resident_partition_chosen_for_decode_workloads(shim):
    # q_proj, k/v projections and the alignment sweep fit the resident kernel
    for K, r, N in [(4096, 1637, 4096), (4096, 817, 1024), (4096, 1000, 4096), (4096, 1100, 3999)]:
        assert _part(shim, K, r, N)[4] == 1, (K, r, N)
    # MLP projections are too large per workgroup: streaming kernel
    for K, r, N in [(4096, 2867, 14336), (14336, 2867, 4096)]:
        assert _part(shim, K, r, N)[4] == 0, (K, r, N)
    # K not a multiple of 8: streaming kernel
    assert _part(shim, 4100, 100, 512)[4] == 0


def test_decode_partition_balances_q_proj(shim):
    Jw, S, ktps, ntps, kind, js_w, nt_w = _part(shim, 4096, 1637, 4096, allow_res=False)
    assert Jw == 14
    # per-workgroup element count is within 25% of the ideal even split
    per_wg = ktps * 32 * 120 + ntps * 120 * 120
    ideal = (128 * 32 * 120 + 35 * 120 * 120) / S
    assert per_wg <= 1.25 * ideal
