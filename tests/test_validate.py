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
int t_check_group(int n, const long long* K, const long long* r, const long long* N, const unsigned long long* A,
                  const unsigned long long* B, unsigned long long X, const unsigned long long* Y, long long M) {
  char err[256];
  lrv::Shape s[8];
  const void* ys[8];
  for (int i = 0; i < n && i < 8; ++i) {
    s[i] = lrv::Shape{K[i], r[i], N[i], 64, (const void*)A[i], (const void*)B[i]};
    ys[i] = (const void*)Y[i];
  }
  return lrv::check_group(s, n, (const void*)X, ys, M, err, sizeof err);
}
int t_choose_dense(long long K, long long r, long long N, unsigned flags) {
  return lrv::choose_dense(K, r, N, flags) ? 1 : 0;
}
void t_partition(long long K, long long r, long long N, int budget, int allow_res, int* out) {
  lrv::DecPart p = lrv::decode_partition(K, r, N, budget, allow_res != 0);
  out[0] = p.Jw; out[1] = p.S; out[2] = p.ktps; out[3] = p.ntps;
  out[4] = p.kind; out[5] = p.js_w; out[6] = p.nt_w;
}
int t_split_partition(long long K, long long r, long long N, int budget, int* out) {
  lrv::DecPart p{};
  const bool ok = lrv::decode_split_partition(K, r, N, budget, &p);
  out[0] = p.ga; out[1] = p.gn; out[2] = p.gb; out[3] = p.gpw; out[4] = p.ntps; out[5] = p.kind;
  return ok ? 1 : 0;
}
int t_split_stream_partition(long long K, long long r, long long N, int budget, long long max_M, int* out) {
  lrv::DecPart p{};
  const bool ok = lrv::decode_split_stream_partition(K, r, N, budget, &p, 16, max_M);
  out[0] = p.ga; out[1] = p.gn; out[2] = p.gb; out[3] = p.g; out[4] = p.nt; out[5] = p.ntps; out[6] = p.kind;
  return ok ? 1 : 0;
}
int t_split_flat_partition(long long K, long long r, long long N, int budget, long long max_M, int* out) {
  lrv::DecPart p{};
  const bool ok = lrv::decode_split_flat_partition(K, r, N, budget, &p, 16, max_M);
  out[0] = p.ga; out[1] = p.gn; out[2] = p.g; out[3] = p.maxc; out[4] = p.ntps; out[5] = p.kind;
  return ok ? 1 : 0;
}
void t_partition2(long long K, long long r, long long N, int budget, int allow_res, int split, long long max_M,
                  int* out) {
  lrv::DecPart p = lrv::decode_partition(K, r, N, budget, allow_res != 0, split != 0, max_M);
  out[0] = p.Jw; out[1] = p.S; out[2] = p.ktps; out[3] = p.ntps;
  out[4] = p.kind; out[5] = p.js_w; out[6] = p.nt_w;
}
void t_prefill_plan(long long rows, long long c0, long long c1, int nout, long long kd, int cus, int kinds,
                    int* out) {
  const int64_t cols[2] = {c0, c1};
  lrv::PrePlan p = lrv::prefill_plan(rows, cols, nout, kd, cus, 32, kinds);
  out[0] = p.nb; out[1] = p.splits; out[2] = p.split_steps; out[3] = p.kind;
}
int t_xcd_plan(long long K, long long r, long long N, int pn, long long max_M, long long* out) {
  lrv::XcdPlan p{};
  const bool ok = lrv::xcd_plan(K, r, N, pn, max_M, &p);
  const long long v[14] = {p.pn, p.pa, p.rs, p.nc, p.cpr_a, p.cpr_b, p.da, p.db, p.ldtp, p.ws,
                           (long long)p.lds, (long long)p.tpart_bytes, (long long)p.tfin_bytes, (long long)p.ypart_bytes};
  for (int i = 0; i < 14; ++i) out[i] = v[i];
  return ok ? 1 : 0;
}
long long t_partial_bytes(long long max_M, long long K, long long r_pad, long long N, int cus) {
  return lrv::prefill_partial_bytes(max_M, K, r_pad, N, cus);
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
    P = ctypes.POINTER
    lib.t_check_group.argtypes = [ctypes.c_int, P(ll), P(ll), P(ll), P(ull), P(ull), ull, P(ull), ll]
    lib.t_choose_dense.argtypes = [ll, ll, ll, ctypes.c_uint]
    lib.t_partition.argtypes = [ll, ll, ll, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.t_prefill_plan.argtypes = [ll, ll, ll, ctypes.c_int, ll, ctypes.c_int, ctypes.c_int, ctypes.POINTER(ctypes.c_int)]
    lib.t_xcd_plan.argtypes = [ll, ll, ll, ctypes.c_int, ll, ctypes.POINTER(ll)]
    lib.t_partial_bytes.argtypes = [ll, ll, ll, ll, ctypes.c_int]
    lib.t_partial_bytes.restype = ll
    return lib


OK, INVALID, UNSUPPORTED = 0, 1, 2
MB = 1 << 20


def _group(shim, K, r, N, A, B, X, Y, M=4):
    n = len(K)
    ll, ull = ctypes.c_longlong, ctypes.c_ulonglong
    arr = lambda t, v: (t * 8)(*v)
    return shim.t_check_group(n, arr(ll, K), arr(ll, r), arr(ll, N), arr(ull, A), arr(ull, B), X, arr(ull, Y), M)


def test_group_validation(shim):
    # q, k, v: equal K, different r and N
    K, r, N = [64, 64, 64], [13, 7, 7], [64, 16, 16]
    A = [10 * MB, 11 * MB, 12 * MB]
    B = [13 * MB, 14 * MB, 15 * MB]
    X, Y = 20 * MB, [30 * MB, 40 * MB, 50 * MB]
    assert _group(shim, K, r, N, A, B, X, Y) == OK
    assert _group(shim, K[:1], r[:1], N[:1], A, B, X, Y) == OK
    assert _group(shim, K + [64], r + [5], N + [8], A + [16 * MB], B + [17 * MB], X, Y + [60 * MB]) == OK
    # n outside 1..4
    assert _group(shim, [], [], [], [], [], X, []) == INVALID
    assert _group(shim, K + K[:2], r + r[:2], N + N[:2], A + A[:2], B + B[:2], X, Y + Y[:2]) == INVALID
    # unequal K
    assert _group(shim, [64, 64, 32], r, N, A, B, X, Y) == INVALID
    # output 2 overlaps output 0 (q writes 4 x 64 bf16 = 512 bytes from Y[0])
    assert _group(shim, K, r, N, A, B, X, [Y[0], Y[1], Y[0] + 256]) == INVALID
    assert _group(shim, K, r, N, A, B, X, [Y[0], Y[1], Y[0] + 512]) == OK
    # an output overlaps another projection's factor, or X
    assert _group(shim, K, r, N, A, B, X, [Y[0], B[2] + 2, Y[2]]) == INVALID
    assert _group(shim, K, r, N, A, B, X, [Y[0], Y[1], X + 16]) == INVALID
    # bad M for every projection; M == 0 skips the overlap checks
    assert _group(shim, K, r, N, A, B, X, Y, M=65) == INVALID
    assert _group(shim, K, r, N, A, B, X, [Y[0], Y[0], Y[0]], M=0) == OK


def test_create_validation(shim):
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 0) == OK
    assert shim.t_check_create(4096, 1637, 4096, 0, 0x2000000, 16, 0) == INVALID
    assert shim.t_check_create(4096, 0, 4096, 0x100000, 0x2000000, 16, 0) == INVALID
    assert shim.t_check_create(4096, 1637, 4096, 0x100008, 0x2000000, 16, 0) == INVALID  # 8B aligned only
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 1024) == UNSUPPORTED  # unknown flag
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 512) == OK  # DECODE_XCD
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 512 | 128) == INVALID  # XCD | SPLIT
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 512 | 4) == INVALID  # XCD | STREAMING
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 256) == OK  # DECODE_RESIDENT
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 384) == INVALID  # SPLIT | RESIDENT
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 260) == INVALID  # STREAMING | RESIDENT
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 128) == OK  # DECODE_SPLIT
    # DECODE_SPLIT handles are decode-only (their copy of A and B is what decode reads)
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 17, 128) == INVALID
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 8, 128 | 2) == INVALID
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 132) == INVALID  # with STREAMING
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 32) == OK  # DENSE
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 64) == OK  # FACTORED
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 96) == INVALID  # both
    # DENSE needs W = A.B (K x N bf16) inside a 32-bit range; the factors alone fit
    assert shim.t_check_create(40000, 8, 40000, 0x100000, 0x2000000, 16, 32) == UNSUPPORTED
    assert shim.t_check_create(40000, 8, 40000, 0x100000, 0x2000000, 16, 0) == OK
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 4096, 8) == OK      # PREFILL_TWO_WAVE
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 4096, 16) == OK     # PREFILL_ONE_WAVE
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 4096, 24) == INVALID  # both
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 16, 4) == OK
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 17, 1) == UNSUPPORTED
    assert shim.t_check_create(4096, 1637, 4096, 0x100000, 0x2000000, 17, 2) == OK
    assert shim.t_check_create(1 << 25, 8, 8, 0x100000, 0x2000000, 1, 0) == INVALID


def test_dense_fallback_choice(shim):
    # taken when the factors hold >= 95% of the dense matrix's bytes:
    # r (K + N) >= 0.95 K N, or when forced; never with FACTORED
    assert shim.t_choose_dense(4096, 817, 1024, 0) == 1     # k/v: 99.7%
    assert shim.t_choose_dense(4096, 1637, 4096, 0) == 0    # q/o: 80%
    assert shim.t_choose_dense(4096, 2867, 14336, 0) == 0   # gate/up: 90%
    assert shim.t_choose_dense(14336, 2867, 4096, 0) == 0   # down: 90%
    assert shim.t_choose_dense(4096, 1100, 3999, 0) == 0    # sweep
    assert shim.t_choose_dense(512, 107, 512, 0) == 0       # tiny config
    assert shim.t_choose_dense(512, 250, 512, 0) == 1       # 97.7%
    assert shim.t_choose_dense(512, 243, 512, 0) == 0       # 94.9%
    assert shim.t_choose_dense(512, 244, 512, 0) == 1       # 95.3%
    assert shim.t_choose_dense(4096, 1637, 4096, 32) == 1   # forced
    assert shim.t_choose_dense(4096, 817, 1024, 64) == 0    # FACTORED
    assert shim.t_choose_dense(40000, 39999, 40000, 0) == 0  # W past a 32-bit range
    # the rule against exact integers
    for K, r, N in [(7, 3, 5), (100, 49, 100), (100, 48, 100), (33, 40, 17)]:
        assert shim.t_choose_dense(K, r, N, 0) == int(100 * r * (K + N) >= 95 * K * N)


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


def _split(shim, K, r, N, budget=256):
    out = (ctypes.c_int * 6)()
    ok = shim.t_split_partition(K, r, N, budget, out)
    return ok, tuple(out)


@pytest.mark.parametrize("K,r,N", [(4096, 1637, 4096), (4096, 1000, 4096), (4096, 1100, 3999), (4096, 817, 1024),
                                   (33, 5, 7), (100, 17, 121), (257, 241, 3999), (8, 1, 1), (4096, 1, 4096),
                                   (4096, 2048, 2048)])
def test_split_partition_covers_and_fits(shim, K, r, N):
    ok, (ga, gn, gb, gpw, per, kind) = _split(shim, K, r, N)
    assert ok and kind == 2
    assert ga == -(-r // 16) and gn == -(-N // 16)
    assert gpw in (1, 2, 4, 8) and gb == -(-gn // gpw)   # every column group has a producer
    assert ga + gb <= 256                                # one launch, every workgroup resident
    nkb = -(-r // 32)
    assert per == -(-nkb // (8 // gpw)) and per <= 16    # B blocks held per wave
    assert (8 // gpw) * per >= nkb                       # the waves of a group cover the rank
    # the smallest gpw that fits
    if gpw > 1:
        g2 = gpw // 2
        assert ga + -(-gn // g2) > 256 or -(-nkb // (8 // g2)) > 16


def test_split_partition_q_proj_and_limits(shim):
    ok, (ga, gn, gb, gpw, per, _) = _split(shim, 4096, 1637, 4096)
    assert ok and (ga, gn, gb, gpw, per) == (103, 256, 128, 2, 13)
    # MLP projections: too many producers, or too many B blocks per wave
    assert not _split(shim, 4096, 2867, 14336)[0]
    assert not _split(shim, 14336, 2867, 4096)[0]
    # a rank that needs more than 16 blocks per wave even at gpw = 1
    assert not _split(shim, 4096, 4200, 512)[0]
    # a small machine
    assert not _split(shim, 4096, 1637, 4096, budget=64)[0]


def test_split_flag_selects_split_partition(shim):
    out = (ctypes.c_int * 7)()
    shim.t_partition2(4096, 1637, 4096, 256, 1, 1, ctypes.c_longlong(16), out)
    assert out[4] == 2
    shim.t_partition2(4096, 4200, 14336, 256, 1, 1, ctypes.c_longlong(16), out)   # fits neither split kind: the other kinds
    assert out[4] in (0, 1)
    shim.t_partition2(4096, 1637, 4096, 256, 1, 0, ctypes.c_longlong(16), out)
    assert out[4] == 1


def _split_stream(shim, K, r, N, budget=256, max_M=1):
    out = (ctypes.c_int * 7)()
    ok = shim.t_split_stream_partition(K, r, N, budget, max_M, out)
    return ok, tuple(out)


@pytest.mark.parametrize("K,r,N,max_M", [(4096, 2867, 14336, 1), (4096, 2867, 14336, 8), (2048, 2867, 14336, 1),
                                         (1001, 2500, 9001, 3), (2048, 2000, 12000, 12), (512, 4096, 64, 1),
                                         (2048, 1637, 4096, 1), (1024, 700, 30000, 2)])
def test_split_stream_partition_covers_and_balances(shim, K, r, N, max_M):
    ok, (ga, gn, gy, g, nt, per, kind) = _split_stream(shim, K, r, N, max_M=max_M)
    assert ok and kind == 3
    assert ga == -(-r // 16) and gn == -(-N // 16) and g == min(256, ga + gn) and gy == g - ga
    nkb = -(-r // 32)
    assert per == -(-nkb // 8) and per <= 16 and (max_M <= 8 or per <= 8)
    if gy == 0:
        assert ga * nt >= gn                 # T producers take every group
    else:
        assert 0 <= ga * nt <= gn            # the rest go to the Y-only workgroups
        # bytes per workgroup balanced to within one group (or T producers
        # take none because their A slab alone exceeds the average)
        ca = -(-K // 32) + max_M * K * 2 / 1024.0
        rest = gn - ga * nt
        y_max = -(-rest // gy) * nkb
        t_bytes = ca + nt * nkb
        assert ca <= (ga * ca + gn * nkb) / g    # T producers not above the average
        assert nt == 0 or t_bytes <= y_max + 2 * nkb + ca


def test_split_stream_partition_layer_shapes(shim):
    # gate/up at M = 1: 180 T producers with 3 column groups each, 76 more
    # workgroups share the other 356
    ok, (ga, gn, gy, g, nt, per, _) = _split_stream(shim, 4096, 2867, 14336)
    assert ok and (ga, gn, gy, g, nt, per) == (180, 896, 76, 256, 3, 12)
    # down: the A slab (448 KB) exceeds the average share: not this kind
    assert not _split_stream(shim, 14336, 2867, 4096)[0]
    # M up to 16 needs at most 8 blocks per wave
    assert not _split_stream(shim, 4096, 2867, 14336, max_M=16)[0]
    # a rank above 4096 does not fit; more T producers than CUs neither
    assert not _split_stream(shim, 4096, 4200, 512)[0]
    assert not _split_stream(shim, 4096, 4100, 4096, budget=200)[0]


def _split_flat(shim, K, r, N, budget=256, max_M=1):
    out = (ctypes.c_int * 6)()
    ok = shim.t_split_flat_partition(K, r, N, budget, max_M, out)
    return ok, tuple(out)


@pytest.mark.parametrize("K,r,N,budget", [(14336, 2867, 4096, 256), (12001, 2000, 6000, 256), (12000, 1800, 9000, 256),
                                          (4096, 1637, 4096, 256), (300, 700, 50, 256), (14336, 2867, 4096, 200)])
def test_split_flat_partition_contributors_fit(shim, K, r, N, budget):
    ok, (ga, gn, g, maxc, per, kind) = _split_flat(shim, K, r, N, budget=budget)
    assert ok and kind == 4 and g == budget
    nka = -(-K // 32)
    tb = ga * nka
    # every workgroup's share of the slice-major blocks spans at most two
    # slices, and every slice has at most maxc contributors
    lo = [w * tb // g for w in range(g + 1)]
    assert tb >= g                           # no workgroup's share is empty
    for w in range(g):
        assert lo[w] < lo[w + 1]
        assert (lo[w + 1] - 1) // nka - lo[w] // nka <= 1
    for j in range(ga):
        contrib = [w for w in range(g) if lo[w] < lo[w + 1] and lo[w] < (j + 1) * nka and lo[w + 1] > j * nka]
        assert 1 <= len(contrib) <= maxc
        # the owner (first contributor) is the one flat_owner finds for the slice's first block
        b = j * nka
        assert contrib[0] == ((b + 1) * g + tb - 1) // tb - 1


def test_split_flat_partition_rejects_empty_shares(shim):
    # fewer A blocks than workgroups: some shares would be empty
    assert not _split_flat(shim, 100, 300, 50)[0]          # 19 slices x 4 blocks = 76 < 256
    assert _split_flat(shim, 100, 300, 50, budget=64)[0]   # 76 >= 64


def test_decode_partition_prefers_register_split_then_streaming_split(shim):
    out = (ctypes.c_int * 7)()
    shim.t_partition2(4096, 1637, 4096, 256, 1, 1, ctypes.c_longlong(16), out)
    assert out[4] == 2
    shim.t_partition2(4096, 2867, 14336, 256, 1, 1, ctypes.c_longlong(1), out)   # B too large for registers: streaming split
    assert out[4] == 3
    shim.t_partition2(14336, 2867, 4096, 256, 1, 1, ctypes.c_longlong(1), out)   # A-heavy (down): flat split
    assert out[4] == 4
    shim.t_partition2(14336, 2867, 4096, 256, 1, 0, ctypes.c_longlong(1), out)   # resident/streaming only
    assert out[4] in (0, 1)


TWO_WAVE, ONE_WAVE = 1, 2


def _plan(shim, rows, cols, kd, cus=256, kinds=TWO_WAVE):
    out = (ctypes.c_int * 4)()
    c = list(cols) + [0]
    shim.t_prefill_plan(rows, c[0], c[1], len(cols), kd, cus, kinds, out)
    return tuple(out)


PLAN_SHAPES = [
    (4096, (2880,), 4096), (4096, (14336,), 2880),          # MLP up-projection, both phases
    (2048, (1664,), 4096), (2048, (4096,), 1664),           # q_proj at M = 2048
    (2048, (2880, 2880), 4096), (2048, (14336, 14336), 2880),  # packed gate/up
    (512, (1056,), 4096), (512, (3999,), 1056),             # alignment sweep at M = 512
    (17, (128,), 512), (40, (512,), 128), (300, (33,), 7),  # small and ragged
]


@pytest.mark.parametrize("kinds", [TWO_WAVE, ONE_WAVE, TWO_WAVE | ONE_WAVE])
@pytest.mark.parametrize("rows,cols,kd", PLAN_SHAPES)
def test_prefill_plan_covers_k_and_fits(shim, rows, cols, kd, kinds):
    nb, splits, steps, kind = _plan(shim, rows, cols, kd, kinds=kinds)
    nks = -(-kd // 32)
    assert kind in (0, 1) and (kinds >> kind) & 1
    if kind == 0:
        assert nb in (2, 3, 4, 6, 7)
    else:
        # the one-wave kernel: 256-wide tiles, splits on 64-deep stages
        assert nb == 8 and steps % 2 == 0
    assert splits >= 1 and steps >= 1
    # every k-step is in exactly one split and no split is empty
    assert splits * steps >= nks and (splits - 1) * steps < nks


def test_prefill_plan_picks_by_cost(shim):
    both = TWO_WAVE | ONE_WAVE
    # MLP up, both phases (whatever r mod 8 is): the two-wave kernel, 192
    # columns wide for phase 1 (240 tiles: one round), 224 for phase 2 (1024
    # tiles: four full rounds, where the one-wave kernel's 896 leave the
    # last round half empty)
    assert _plan(shim, 4096, (14336,), 2880, kinds=both)[::3] == (7, 0)
    assert _plan(shim, 4096, (2880,), 4096, kinds=both)[::3] == (6, 0)
    # only one kind allowed: that kind
    assert _plan(shim, 4096, (14336,), 2880, kinds=TWO_WAVE)[3] == 0
    assert _plan(shim, 4096, (2880,), 4096, kinds=ONE_WAVE)[3] == 1


def test_prefill_plan_does_not_depend_on_alignment(shim):
    # the plan sees only the padded rank, the output width and the depth:
    # every r in 2864..2872 (all residues mod 8) and widths 3993..4000 get
    # the plan of their aligned neighbour
    both = TWO_WAVE | ONE_WAVE
    p1 = {_plan(shim, 4096, (-(-r // 32) * 32,), 4096, kinds=both) for r in range(2849, 2881)}
    assert len(p1) == 1
    p2 = {_plan(shim, 4096, (n,), 2880, kinds=both)[:2] for n in range(3969, 4001)}
    assert len(p2) == 1


def test_prefill_plan_fills_the_machine_for_small_m(shim):
    # MLP up at M = 4096: enough tiles, no split
    assert _plan(shim, 4096, (14336,), 2880)[1] == 1
    # the M = 512 sweep shape has 12 tiles of 256 x 192: it splits k
    nb, splits, steps, kind = _plan(shim, 512, (1056,), 4096)
    tiles = 2 * -(-1056 // (32 * nb))
    assert splits > 1 and tiles * splits >= 64


def test_prefill_partial_bytes_cover_every_plan(shim):
    for max_M, K, r_pad, N in [(4096, 4096, 2880, 14336), (2048, 4096, 1664, 4096), (512, 4096, 1056, 3999),
                               (600, 14336, 2880, 4096)]:
        have = shim.t_partial_bytes(max_M, K, r_pad, N, 256)
        for M in list(range(17, max_M + 1, 97)) + [max_M]:
            for cols, kd in (((r_pad,), K), ((N,), r_pad)):
                for kinds in (TWO_WAVE, ONE_WAVE, TWO_WAVE | ONE_WAVE):
                    nb, splits, steps, kind = _plan(shim, M, cols, kd, kinds=kinds)
                    if splits > 1:
                        assert splits * M * (-(-cols[0] // 4) * 4) * 4 <= have, (max_M, M, cols, kd, splits)


def _xcd(shim, K, r, N, pn, max_M):
    out = (ctypes.c_longlong * 14)()
    ok = shim.t_xcd_plan(K, r, N, pn, max_M, out)
    keys = ["pn", "pa", "rs", "nc", "cpr_a", "cpr_b", "da", "db", "ldtp", "ws", "lds", "tpart", "tfin", "ypart"]
    return bool(ok), dict(zip(keys, out))


def _inst(cpr):
    # 64-lane DMA instructions per 32-row k-step tile with rows of cpr + 1 chunks
    return (32 * (cpr + 1) + 63) // 64


@pytest.mark.parametrize("K,r,N", [(4096, 1637, 4096), (4096, 2867, 14336), (14336, 2867, 4096), (1024, 300, 1000),
                                   (4096, 1024, 4096), (4096, 1063, 3999), (2048, 7, 33), (333, 2049, 77)])
@pytest.mark.parametrize("pn", [8, 16, 32])
@pytest.mark.parametrize("max_M", [1, 8, 16])
def test_xcd_plan_covers_and_fits(shim, K, r, N, pn, max_M):
    ok, p = _xcd(shim, K, r, N, pn, max_M)
    if not ok:
        return
    rw = -(-r // 8)
    assert 1 <= p["pa"] < pn and p["pa"] % p["rs"] == 0 and p["rs"] & (p["rs"] - 1) == 0
    sub = -(-rw // p["rs"])                      # rank columns of one A workgroup's sub-range
    assert 8 * p["cpr_a"] >= sub and p["cpr_a"] % 2 == 0 and p["cpr_a"] <= 32
    assert p["ws"] * (pn - p["pa"]) >= N         # the B slabs cover N
    assert p["nc"] in (1, 2, 4, 8) and 8 * p["cpr_b"] * p["nc"] >= p["ws"] and p["cpr_b"] <= 32
    assert p["ldtp"] >= rw and p["lds"] <= 160 * 1024
    assert p["da"] >= 1 and p["da"] * (_inst(p["cpr_a"]) + 1) <= 62
    assert p["db"] >= 1 and p["db"] * _inst(p["cpr_b"]) <= 62
    colb = 16 * -(-max_M // 4)
    assert p["tfin"] == 8 * p["ldtp"] * colb
    assert p["ypart"] == 8 * (pn - p["pa"]) * p["ws"] * colb


def test_xcd_plan_layer_shapes(shim):
    # every projection of the layer has a plan for the whole device and for
    # half of it (two projections sharing a launch)
    for K, r, N in [(4096, 1637, 4096), (4096, 2867, 14336), (14336, 2867, 4096)]:
        for pn in (32, 16):
            ok, p = _xcd(shim, K, r, N, pn, 8)
            assert ok, (K, r, N, pn)
    ok, p = _xcd(shim, 4096, 1637, 4096, 32, 8)
    assert (p["pa"], p["rs"], p["nc"]) == (16, 1, 1)
    # too few workgroups for the up-projection's B slab
    assert not _xcd(shim, 4096, 2867, 14336, 8, 1)[0]
    assert not _xcd(shim, 4096, 1637, 4096, 1, 1)[0]
