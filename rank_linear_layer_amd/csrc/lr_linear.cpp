// C-ABI host library of the factorized linear layer (see include/lr_linear.h).
//
// Owns: argument validation (lr_validate.h), the per-shape partition chosen
// at create time, the device workspace, and kernel launches on the caller's
// stream.  Every step of Y = (X.A).B runs in the HIP kernels of
// lr_decode.hip and lr_prefill.hip; nothing here computes on the host.
#include <hip/hip_runtime.h>

#include <stdarg.h>
#include <stdio.h>
#include <string.h>

#include <atomic>
#include <mutex>
#include <new>

#include "../../include/lr_linear.h"
#include "lr_kernels.h"
#include "lr_validate.h"

namespace {

thread_local char g_err[512] = "";

lr_status fail(lr_status st, const char* fmt, ...) __attribute__((format(printf, 2, 3)));
lr_status fail(lr_status st, const char* fmt, ...) {
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(g_err, sizeof g_err, fmt, ap);
  va_end(ap);
  return st;
}

lr_status hip_fail(hipError_t e, const char* what) {
  return fail(LR_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
}

}  // namespace

// The library's other translation units report through the same
// thread-local detail string (not exported).
__attribute__((visibility("hidden"))) lr_status lr_internal_fail(lr_status st, const char* msg) {
  return fail(st, "%s", msg);
}

namespace {

constexpr size_t kAlign = 256;
// Replicas of the role-split kernels' T planes and flags: the Y producers'
// reads of the same few kilobytes spread over this many copies.
#ifndef LR_SPLIT_NREP
#define LR_SPLIT_NREP 8
#endif
constexpr int kSplitReplicas = LR_SPLIT_NREP;
inline size_t align_up(size_t x) { return (x + kAlign - 1) / kAlign * kAlign; }

}  // namespace

struct lr_linear {
  int64_t K, r, N, max_M, r_pad;
  uint32_t flags;
  int device;
  const uint16_t* A;
  const uint16_t* B;
  // workspace
  void* ws;
  size_t ws_bytes;
  // decode partition and workspace views
  bool has_decode;
  lrv::DecPart dp;
  int dec_max_M;
  char* dws;          // decode workspace base
  int64_t dws_bytes;
  uint32_t* ctrl;
  uint32_t* tcnt;
  uint32_t* tflag;
  uint32_t* ycnt;
  uint32_t off_tpart, off_tfin, off_ypart, off_tflag, off_yflag;
  // register-streaming kernel: a second plan on half the compute units, so
  // that two such projections sharing X (gate and up) fit one launch; its
  // tables share the decode region (same control words)
  bool has_half;
  lrv::DecPart dph;
  uint32_t hoff_tpart, hoff_ypart;
  bool xcd_local;
  // prefill workspace: T [max_M x r_pad] bf16, and fp32 k-split partials
  bool has_prefill;
  uint16_t* Tbuf;
  float* part;
  int64_t part_bytes;
  // plan of the last prefill call per phase: kernel kind, nb, splits (reported by describe)
  mutable std::atomic<int> last_plan[2][3];
  // dense fallback: W = A.B row-major [K x N] (prefill) and in the decode
  // layout (decode), both formed at create
  bool dense;
  uint16_t* W;
  uint16_t* Wsw;
  float* dpart;     // dense decode: [kDenseMaxSplits][ceil(N/16)][256] fp32 partials
  uint32_t* dcnt;   // dense decode: [ceil(N/16)] arrival counters
  // role-split decode (dp.kind 2): A and B in the operand block layout,
  // T [dec_max_M x 32 ceil(r/32)] fp32 and the T slice flags
  uint16_t* Asw;
  uint16_t* Bsw;
  uint16_t* Tsp;
  uint32_t* sflags;
  int nrep, ldf;       // replicas of T and of its flags; flag words per replica
  float* fpart;        // flat variant: partial tiles [GA][maxc] of 16 x 16 fp32
  uint32_t* pflags;    // flat variant: their flags
  // XCD-sliced decode (dp.kind 5, LR_FLAG_DECODE_XCD): plans for xcd_P, xcd_P / 2
  // and xcd_P / 4 workgroups per XCD (alone in a launch, or one of two, or
  // of three or four projections sharing X), and their exchange tables
  int xcd_P;
  bool xcd_ok[3];
  lrv::XcdPlan xp[3];
  uint32_t* xflags;  // [3][8 xcd_P] epoch stamps
  float* xtpart;
  float* xtfin;
  float* xypart;
  uint32_t spin_limit;  // polls before a cross-workgroup wait gives up
  uint32_t stall_xor;   // LR_FLAG_TEST_STALL: kStallXor (the T hand-off wait cannot succeed), else 0
  // pinned host word that a decode kernel raises when one of its waits gave
  // up; the next call on the handle (or lr_linear_status) reports it
  uint32_t* err_host;
  uint32_t* err_dev;
};

namespace {

bool use_decode(const lr_linear* h, int64_t M) {
  if (h->flags & LR_FLAG_FORCE_DECODE) return true;
  if (h->flags & LR_FLAG_FORCE_PREFILL) return false;
  return M <= LR_DECODE_MAX_M;
}

// Fill the kernel-side descriptor of one projection in a decode launch.
lrk::DecProj dec_proj(const lr_linear* h, uint16_t* Y, int wg_begin, bool half = false) {
  lrk::DecProj p;
  p.A = h->A;
  p.B = h->B;
  p.Y = Y;
  p.ws = h->dws;
  p.ws_bytes = h->dws_bytes;
  p.ctrl = h->ctrl;
  p.tcnt = h->tcnt;
  p.tflag = h->tflag;
  p.ycnt = h->ycnt;
  p.off_tpart = h->off_tpart;
  p.off_tfin = h->off_tfin;
  p.off_ypart = h->off_ypart;
  p.off_tflag = h->off_tflag;
  p.off_yflag = h->off_yflag;
  p.js_w = h->dp.js_w;
  // the XCD-local exchange needs workgroup (local id) on XCD local % 8
  p.xcd_local = (h->xcd_local && wg_begin % 8 == 0) ? 1 : 0;
  p.r = (int)h->r;
  p.N = (int)h->N;
  const lrv::DecPart& dp = half ? h->dph : h->dp;
  p.Jw = dp.Jw;
  p.S = dp.S;
  p.ktps = dp.ktps;
  p.ntps = dp.ntps;
  if (half) {
    p.off_tpart = h->hoff_tpart;
    p.off_ypart = h->hoff_ypart;
  }
  p.wg_begin = wg_begin;
  p.err = h->err_dev;
  p.spin_limit = h->spin_limit;
  p.stall_xor = h->stall_xor;
  return p;
}

// Frees what a partly built handle holds (create's error paths).
void discard(lr_linear* h) {
  if (h->err_host) (void)hipHostFree(h->err_host);
  if (h->ws) (void)hipFree(h->ws);
  delete h;
}

// Whether workgroups are dealt to XCDs round-robin (checked once per device).
bool xcd_map_ok(int device) {
  static std::mutex mu;
  static int cached[64];
  static bool init = false;
  std::lock_guard<std::mutex> lock(mu);
  if (!init) {
    for (int& c : cached) c = -1;
    init = true;
  }
  if (device < 0 || device >= 64) return false;
  if (cached[device] < 0) cached[device] = lrk::xcd_round_robin(1024) ? 1 : 0;
  return cached[device] == 1;
}

// Byte offsets of the in-place decode kernels' regions (LDS-resident and
// register-streaming, dp.kind 1 and 0) in a workspace whose decode part
// starts at `off`.  The control words (ctrl, counters, flags) come first and
// end where the fp32 tables begin (`tpart`).
struct InplaceLayout {
  size_t ctrl, tcnt, tflag, yflag, ycnt, tpart, tfin, ypart, end;
};
InplaceLayout inplace_layout(const lrv::DecPart& dp, int max_M, size_t off) {
  const int64_t G = (int64_t)dp.Jw * dp.S;
  InplaceLayout L;
  L.ctrl = off;
  off = align_up(off + 64);
  L.tcnt = off;
  off = align_up(off + (size_t)dp.Jw * 4);
  L.tflag = off;
  off = align_up(off + (size_t)G * 4);  // one flag per workgroup (resident kernel) or per slice
  L.yflag = off;
  off = align_up(off + (size_t)G * 4);
  L.ycnt = off;
  off = align_up(off + (size_t)dp.S * 4);
  // T partials of the streaming kernel and Y partials of both are stored as
  // epoch-tagged exchange words: each value beside a tag, twice the bytes
  L.tpart = off;
  off = align_up(off + (size_t)G * max_M * (dp.kind == 1 ? 128 * 4 : dp.js_w * 8));
  L.tfin = off;
  off = align_up(off + (size_t)dp.Jw * max_M * dp.js_w * 4);
  L.ypart = off;
  off = align_up(off + (size_t)G * dp.ntps * max_M * dp.nt_w * 8);
  L.end = off;
  return L;
}

int num_cus(int device) {
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, device) != hipSuccess || cus <= 0) cus = 256;
  return cus;
}

#ifdef LR_DECODE_TRACE
uint64_t* g_trace = nullptr;
bool g_xcd_coherent = false;  // trace builds: run the XCD-local exchange device-coherent
#endif

// Dense-fallback decode of n <= kDenseMaxOut projections sharing X (equal
// K) in one launch.
lr_status run_dense_decode(const lr_linear* const* hs, uint16_t* const* Ys, int n, const void* X, int64_t M,
                           hipStream_t stream) {
  lrk::DenseArgs a;
  memset(&a, 0, sizeof a);
  a.X = (const uint16_t*)X;
  a.M = M;
  a.K = hs[0]->K;
  a.nk = lrv::ceil_div(hs[0]->K, 32);
  a.nout = n;
  for (int i = 0; i < n; ++i) {
    a.o[i].Wsw = hs[i]->Wsw;
    a.o[i].Y = Ys[i];
    a.o[i].N = hs[i]->N;
    a.o[i].part = hs[i]->dpart;
    a.o[i].cnt = hs[i]->dcnt;
    a.ng += lrv::ceil_div(hs[i]->N, 16);
  }
  // K slices per column group, measured on MI355X: slicing pays only for
  // deep, narrow outputs (K = 14336, 64 groups: four slices 10.8 us against
  // 14.3), so the slices bring the launch to about one workgroup per compute
  // unit and keep at least 64 k-steps each
  const int64_t want = lrv::ceil_div((int64_t)num_cus(hs[0]->device), a.ng);
  a.splits = (int)std::max<int64_t>(1, std::min<int64_t>({want, (int64_t)lrk::kDenseMaxSplits, a.nk / 64}));
  const hipError_t e = lrk::launch_dense_decode(a, stream);
  if (e != hipSuccess) return hip_fail(e, "dense decode launch");
  return LR_OK;
}

static_assert(lrk::kSplitMaxBlocks == 16 && lrk::kSplitMaxTBytes == 144 * 1024,
              "the split plan (decode_split_partition defaults) matches the kernel's limits");
lr_status run_split_decode(const lr_linear* h, uint16_t* Y, const void* X, int64_t M, hipStream_t stream,
                           bool check_only = false) {
  lrk::SplitArgs a;
  a.err = h->err_dev;
  a.spin_limit = h->spin_limit;
  a.stall_xor = h->stall_xor;
  a.check_only = check_only ? 1 : 0;
  a.X = (const uint16_t*)X;
  a.Asw = h->Asw;
  a.Bsw = h->Bsw;
  a.Y = Y;
  a.P = h->Tsp;
  a.flags = h->sflags;
  a.ctrl = h->ctrl;
  a.nrep = h->nrep;
  a.ldf = h->ldf;
  a.trace = nullptr;
#ifdef LR_DECODE_TRACE
  a.trace = g_trace;
#endif
  a.M = (int)M;
  a.K = (int)h->K;
  a.r = (int)h->r;
  a.N = (int)h->N;
  a.nkA = (int)lrv::ceil_div(h->K, 32);
  a.nkB = (int)lrv::ceil_div(h->r, 32);
  a.ldp = 32 * a.nkB + 8;
  a.GA = h->dp.ga;
  a.GN = h->dp.gn;
  a.GB = h->dp.gb;
  a.gpw = h->dp.gpw;
  a.stream_y = h->dp.kind == 4 ? 2 : h->dp.kind == 3 ? 1 : 0;
  a.G = h->dp.g;
  a.nt = h->dp.nt;
  a.part = h->fpart;
  a.pflags = h->pflags;
  a.maxc = h->dp.maxc;
  const hipError_t e = lrk::launch_decode_split(a, stream);
  if (e == hipErrorCooperativeLaunchTooLarge)
    return fail(LR_ERR_UNSUPPORTED, "split decode: %d workgroups cannot all be resident at once on this device",
                a.stream_y ? a.G : a.GA + a.GB);
  if (e != hipSuccess) return hip_fail(e, "split decode launch");
  return LR_OK;
}

// A decode kernel of an earlier call gave up waiting for another workgroup
// (not every workgroup was resident, e.g. another kernel held compute
// units): that call's output is invalid.  Reported once, then cleared.
lr_status take_stall(const lr_linear* h) {
  if (!h->err_host) return LR_OK;
  if (__atomic_load_n(h->err_host, __ATOMIC_ACQUIRE) == 0) return LR_OK;
  __atomic_store_n(h->err_host, 0u, __ATOMIC_RELEASE);
  return fail(LR_ERR_HIP,
              "an earlier decode call on this handle gave up waiting for another workgroup (the launch's "
              "workgroups were not all resident at once); its output is invalid");
}

// Plan index for pn = xcd_P >> v.
int xcd_share(int n, int rank_by_bytes) {
  if (n == 1) return 0;
  if (n == 2) return 1;
  if (n == 3) return rank_by_bytes == 0 ? 1 : 2;
  return 2;
}

// XCD-sliced decode of n <= kXcdMaxProj kind-5 handles sharing X in one
// launch: projection i takes xcd_P >> v_i workgroups per XCD (all of them
// alone; half each for two; half for the largest of three and a quarter for
// the others; a quarter each for four).  Returns LR_ERR_UNSUPPORTED (with no
// launch) when some handle has no plan for its share.
lr_status run_xcd_decode(const lr_linear* const* hs, uint16_t* const* Ys, int n, const void* X, int64_t M,
                         hipStream_t stream, bool check_only = false) {
  int rank[lrk::kXcdMaxProj] = {0, 0, 0, 0};
  for (int i = 0; i < n; ++i)
    for (int j = 0; j < n; ++j) {
      const int64_t bi = hs[i]->r * (hs[i]->K + hs[i]->N), bj = hs[j]->r * (hs[j]->K + hs[j]->N);
      if (bj > bi || (bj == bi && j < i)) ++rank[i];
    }
  lrk::XcdArgs a;
  memset(&a, 0, sizeof a);
  a.X = (const uint16_t*)X;
  a.M = (int)M;
  a.K = (int)hs[0]->K;
  a.nproj = n;
  a.check_only = check_only ? 1 : 0;
  a.xcd_local = 1;
  a.spin_limit = hs[0]->spin_limit;
#ifdef LR_DECODE_TRACE
  a.trace = g_trace;
#endif
  int p0 = 0;
#ifdef LR_DECODE_TRACE
  const bool force_coherent = g_xcd_coherent;
#else
  const bool force_coherent = false;
#endif
  int64_t lds = 0;
  for (int i = 0; i < n; ++i) {
    const lr_linear* h = hs[i];
    const int v = xcd_share(n, rank[i]);
    if (h->dp.kind != 5 || !h->xcd_ok[v] || h->xcd_P != hs[0]->xcd_P) return LR_ERR_UNSUPPORTED;
    const lrv::XcdPlan& pl = h->xp[v];
    lrk::XcdProj& P = a.p[i];
    P.A = h->A;
    P.B = h->B;
    P.Y = Ys[i];
    P.ctrl = h->ctrl;
    P.err = h->err_dev;
    P.flags = h->xflags;
    P.tpart = h->xtpart;
    P.tfin = h->xtfin;
    P.ypart = h->xypart;
    P.r = (int)h->r;
    P.N = (int)h->N;
    P.p0 = p0;
    P.pn = pl.pn;
    P.pa = pl.pa;
    P.rs = pl.rs;
    P.nc = pl.nc;
    P.cpr_a = pl.cpr_a;
    P.cpr_b = pl.cpr_b;
    P.da = pl.da;
    P.db = pl.db;
    P.ldtp = pl.ldtp;
    P.ws = pl.ws;
    P.stall_xor = h->stall_xor;
    p0 += pl.pn;
    lds = lds > pl.lds ? lds : pl.lds;
    a.xcd_local = a.xcd_local && h->xcd_local;
    a.spin_limit = a.spin_limit < h->spin_limit ? a.spin_limit : h->spin_limit;
  }
  if (p0 != hs[0]->xcd_P) return LR_ERR_UNSUPPORTED;
  if (force_coherent) a.xcd_local = 0;
  a.grid = 8 * p0;
  const hipError_t e = lrk::launch_decode_xcd(a, (int)lds, stream);
  if (e == hipErrorCooperativeLaunchTooLarge)
    return fail(LR_ERR_UNSUPPORTED, "xcd decode: %d workgroups cannot all be resident at once on this device", a.grid);
  if (e != hipSuccess) return hip_fail(e, "xcd decode launch");
  return LR_OK;
}

lr_status run_decode(const lr_linear* const* hs, uint16_t* const* Ys, int n, const void* X, int64_t M,
                     hipStream_t stream, bool check_only = false, bool half = false) {
  if (hs[0]->dp.kind == 5) {
    for (int i = 0; i < n; ++i) {
      const lr_status st = run_xcd_decode(hs + i, Ys + i, 1, X, M, stream, check_only);
      if (st == LR_ERR_UNSUPPORTED) return fail(st, "no XCD-sliced decode plan for this handle");
      if (st != LR_OK) return st;
    }
    return LR_OK;
  }
  if (hs[0]->dp.kind >= 2) {
    for (int i = 0; i < n; ++i) {
      const lr_status st = run_split_decode(hs[i], Ys[i], X, M, stream, check_only);
      if (st != LR_OK) return st;
    }
    return LR_OK;
  }
  lrk::DecArgs a;
  memset(&a, 0, sizeof a);
  a.X = (const uint16_t*)X;
  a.check_only = check_only ? 1 : 0;
#ifdef LR_DECODE_TRACE
  a.trace = g_trace;
#endif
  a.M = (int)M;
  a.K = (int)hs[0]->K;
  a.nproj = n;
  int wg = 0;
  for (int i = 0; i < n; ++i) {
    a.p[i] = dec_proj(hs[i], Ys[i], wg, half);
    const lrv::DecPart& dp = half ? hs[i]->dph : hs[i]->dp;
    wg += dp.Jw * dp.S;
  }
  hipError_t e = hs[0]->dp.kind == 1 ? lrk::launch_decode_res(a, wg, stream) : lrk::launch_decode(a, wg, stream);
  if (e == hipErrorCooperativeLaunchTooLarge)
    return fail(LR_ERR_UNSUPPORTED, "decode: %d workgroups cannot all be resident at once on this device", wg);
  if (e != hipSuccess) return hip_fail(e, "decode launch");
  return LR_OK;
}

// The one-wave-per-SIMD kernel loads P straight into LDS (16-byte aligned
// rows only); its weight loads take any row alignment.
bool w4_operands(const lrk::PreOut& o) {
  return o.ldp % 8 == 0 && reinterpret_cast<uintptr_t>(o.P) % 16 == 0;
}

// Kernel kinds the handles' flags allow for outputs whose operands do (w4)
// or do not suit the one-wave kernel.
int allowed_kinds(const lr_linear* h, bool w4) {
  int kinds = lrv::kPlanTwoWave | (w4 ? lrv::kPlanOneWave : 0);
  if (h->flags & LR_FLAG_PREFILL_TWO_WAVE) kinds = lrv::kPlanTwoWave;
  if ((h->flags & LR_FLAG_PREFILL_ONE_WAVE) && w4) kinds = lrv::kPlanOneWave;
  return kinds;
}

// Plan of one launch over outputs o[0..n), shrunk to one split when a
// handle's partial buffer cannot hold the planned split count.
lrv::PrePlan plan_launch(const lr_linear* const* hs, const lrk::PreArgs& a, int n, int64_t kd, int kinds) {
  const int cus = num_cus(hs[0]->device);
  int64_t cols[lrk::kPreMaxOut] = {};
  for (int i = 0; i < n; ++i) cols[i] = a.o[i].out_cols;
  lrv::PrePlan pl = lrv::prefill_plan(a.rows, cols, n, kd, cus, 32, kinds);
  for (int i = 0; i < n && pl.splits > 1; ++i) {
    const int64_t need = (int64_t)pl.splits * a.rows * lrv::round_up(cols[i], 4) * 4;
    if (need > hs[i]->part_bytes) pl = lrv::prefill_plan(a.rows, cols, n, kd, cus, 1, kinds);
  }
  return pl;
}

lr_status launch_phase(const lr_linear* const* hs, lrk::PreArgs& a, int n, const lrv::PrePlan& pl, int phase,
                       hipStream_t stream, const char* what);

// One prefill phase: C_i = P_i . Q_i for the n outputs in one launch (the
// cost model's kernel and k-split for all of them together), then the
// k-split reduction if the plan splits k.
lr_status prefill_phase(const lr_linear* const* hs, lrk::PreArgs& a, int n, int64_t kd, int phase,
                        hipStream_t stream, const char* what) {
  bool w4 = true;
  for (int i = 0; i < n; ++i) w4 = w4 && w4_operands(a.o[i]);
  const lrv::PrePlan pl = plan_launch(hs, a, n, kd, allowed_kinds(hs[0], w4));
  return launch_phase(hs, a, n, pl, phase, stream, what);
}

lr_status launch_phase(const lr_linear* const* hs, lrk::PreArgs& a, int n, const lrv::PrePlan& pl, int phase,
                       hipStream_t stream, const char* what) {
  int64_t cols[lrk::kPreMaxOut] = {};
  for (int i = 0; i < n; ++i) cols[i] = a.o[i].out_cols;
  for (int i = 0; i < n; ++i) {
    hs[i]->last_plan[phase][0] = pl.kind;
    hs[i]->last_plan[phase][1] = pl.nb;
    hs[i]->last_plan[phase][2] = pl.splits;
  }
  a.nb = pl.nb;
  a.splits = pl.splits;
  a.split_steps = pl.split_steps;
  for (int i = 0; i < n; ++i) {
    a.o[i].col_tiles = (int)lrv::ceil_div(cols[i], 32 * pl.nb);
    a.o[i].part = hs[i]->part;
    a.o[i].ldpart = lrv::round_up(cols[i], 4);
  }
  hipError_t e = pl.kind == 1 ? lrk::launch_prefill_w4(a, stream) : lrk::launch_prefill_gemm(a, stream);
  if (e != hipSuccess) return hip_fail(e, what);
  if (pl.splits > 1) {
    for (int i = 0; i < n; ++i) {
      e = lrk::launch_prefill_reduce(a.o[i].part, pl.splits, a.rows, cols[i], a.o[i].ldpart, a.o[i].C, a.o[i].ldc,
                                     stream);
      if (e != hipSuccess) return hip_fail(e, "prefill k-split reduction launch");
    }
  }
  return LR_OK;
}

lr_status run_prefill(const lr_linear* const* hs, uint16_t* const* Ys, int n, const void* X, int64_t M,
                      hipStream_t stream) {
  // phase 1: T_i = X . A_i, or Y_i = X . W_i for dense-fallback handles
  // (the projections share X in one launch)
  lrk::PreArgs a1;
  memset(&a1, 0, sizeof a1);
  a1.rows = M;
  a1.nout = n;
  a1.row_tiles = (int)lrv::ceil_div(M, lrk::kPreBM);
  for (int i = 0; i < n; ++i) {
    const lr_linear* h = hs[i];
    lrk::PreOut& o = a1.o[i];
    o.P = (const uint16_t*)X;
    o.ldp = h->K;
    o.kd = h->K;
    if (h->dense) {
      o.Q = h->W;
      o.ldq = h->N;
      o.qrows = h->K;
      o.C = Ys[i];
      o.ldc = h->N;
      o.out_cols = h->N;
    } else {
      o.Q = h->A;
      o.ldq = h->r;
      o.qrows = h->K;
      o.C = h->Tbuf;
      o.ldc = h->r_pad;
      o.out_cols = h->r_pad;
    }
  }
  lr_status st = prefill_phase(hs, a1, n, hs[0]->K, 0, stream, "prefill phase-1 launch");
  if (st != LR_OK) return st;
  // phase 2: Y_i = T_i . B_i for the factorized handles
  lrk::PreArgs a2;
  memset(&a2, 0, sizeof a2);
  a2.rows = M;
  a2.row_tiles = a1.row_tiles;
  const lr_linear* h2[lrk::kPreMaxOut];
  int n2 = 0;
  int64_t kd2 = 0;
  for (int i = 0; i < n; ++i) {
    const lr_linear* h = hs[i];
    if (h->dense) continue;
    lrk::PreOut& o = a2.o[n2];
    h2[n2++] = h;
    o.P = h->Tbuf;
    o.ldp = h->r_pad;
    o.kd = h->r_pad;
    o.Q = h->B;
    o.ldq = h->N;
    o.qrows = h->r;
    o.C = Ys[i];
    o.ldc = h->N;
    o.out_cols = h->N;
    kd2 = kd2 > h->r_pad ? kd2 : h->r_pad;
  }
  a2.nout = n2;
  if (n2 == 0) return LR_OK;
  return prefill_phase(h2, a2, n2, kd2, 1, stream, "prefill phase-2 launch");
}

// W = A . B (bf16, row-major [K x N]) with the prefill GEMM (P = A, Q = B,
// one split), then its decode layout when the handle decodes.
lr_status form_dense(lr_linear* h, uint16_t* W) {
  lrk::PreArgs a;
  memset(&a, 0, sizeof a);
  a.rows = h->K;
  a.nout = 1;
  a.row_tiles = (int)lrv::ceil_div(h->K, lrk::kPreBM);
  lrk::PreOut& o = a.o[0];
  o.P = h->A;
  o.ldp = h->r;
  o.kd = h->r;
  o.Q = h->B;
  o.ldq = h->N;
  o.qrows = h->r;
  o.C = W;
  o.ldc = h->N;
  o.out_cols = h->N;
  const bool w4 = w4_operands(o);
  const int kinds = lrv::kPlanTwoWave | (w4 ? lrv::kPlanOneWave : 0);
  const int64_t cols = h->N;
  const lrv::PrePlan pl = lrv::prefill_plan(h->K, &cols, 1, h->r, num_cus(h->device), 1, kinds);
  a.nb = pl.nb;
  a.splits = 1;
  a.split_steps = pl.split_steps;
  o.col_tiles = (int)lrv::ceil_div(cols, 32 * pl.nb);
  o.ldpart = lrv::round_up(cols, 4);
  hipError_t e = pl.kind == 1 ? lrk::launch_prefill_w4(a, nullptr) : lrk::launch_prefill_gemm(a, nullptr);
  if (e != hipSuccess) return hip_fail(e, "dense fallback: W = A.B launch");
  if (h->Wsw) {
    e = lrk::launch_dense_swizzle(W, h->Wsw, h->K, h->N, nullptr);
    if (e != hipSuccess) return hip_fail(e, "dense fallback: decode layout launch");
  }
  e = hipDeviceSynchronize();
  if (e != hipSuccess) return hip_fail(e, "dense fallback: forming W");
  return LR_OK;
}

static_assert(lrk::kDecMaxProj >= lrv::kMaxGroup && lrk::kPreMaxOut >= lrv::kMaxGroup &&
                  lrk::kDenseMaxOut >= lrv::kMaxGroup,
              "group size");
lr_status run_group(const lr_linear* const* hs, uint16_t* const* Ys, int n, const void* X, int64_t M,
                    hipStream_t stream) {
  const lr_linear* dh[lrk::kDecMaxProj];
  uint16_t* dy[lrk::kDecMaxProj];
  const lr_linear* ph[lrk::kPreMaxOut];
  uint16_t* py[lrk::kPreMaxOut];
  const lr_linear* xh[lrk::kDenseMaxOut];  // dense-fallback decode: one launch for all of them
  uint16_t* xy[lrk::kDenseMaxOut];
  int nd = 0, np = 0, nx = 0;
  for (int i = 0; i < n; ++i) {
    if (use_decode(hs[i], M) && hs[i]->dense) {
      xh[nx] = hs[i];
      xy[nx++] = Ys[i];
    } else if (use_decode(hs[i], M)) {
      dh[nd] = hs[i];
      dy[nd++] = Ys[i];
    } else {
      ph[np] = hs[i];
      py[np++] = Ys[i];
    }
  }
  if (nx > 0) {
    const lr_status st = run_dense_decode(xh, xy, nx, X, M, stream);
    if (st != LR_OK) return st;
  }
  {
    // XCD-sliced handles share one launch where every one has a plan for its
    // share of the workgroups; otherwise each runs alone
    const lr_linear* xh5[lrk::kXcdMaxProj];
    uint16_t* xy5[lrk::kXcdMaxProj];
    int n5 = 0, rest = 0;
    for (int i = 0; i < nd; ++i) {
      if (dh[i]->dp.kind == 5) {
        xh5[n5] = dh[i];
        xy5[n5++] = dy[i];
      } else {
        dh[rest] = dh[i];
        dy[rest++] = dy[i];
      }
    }
    nd = rest;
    if (n5 > 0) {
      lr_status st = run_xcd_decode(xh5, xy5, n5, X, M, stream);
      for (int i = 0; st == LR_ERR_UNSUPPORTED && i < n5; ++i) {
        // every kind-5 handle has a plan for running alone
        st = run_xcd_decode(xh5 + i, xy5 + i, 1, X, M, stream);
        if (st == LR_ERR_UNSUPPORTED) return fail(st, "no XCD-sliced decode plan for a handle");
        if (st == LR_OK && i + 1 < n5) st = LR_ERR_UNSUPPORTED;
      }
      if (st != LR_OK) return st;
    }
  }
  for (int b = 0; b < nd;) {
    if (dh[b]->dp.kind >= 2) {  // one launch per projection: it fills the machine
      const lr_status st = run_split_decode(dh[b], dy[b], X, M, stream);
      if (st != LR_OK) return st;
      ++b;
      continue;
    }
    const int per_cu = dh[b]->dp.kind == 1 ? 1 : lrk::decode_blocks_per_cu();
    const int64_t cap = (int64_t)num_cus(dh[b]->device) * per_cu;
    int64_t wgs = (int64_t)dh[b]->dp.Jw * dh[b]->dp.S;
    // two register-streaming projections that do not fit one launch with
    // their own plans share one on their half-machine plans
    if (b + 1 < nd && dh[b]->dp.kind == 0 && dh[b + 1]->dp.kind == 0 && dh[b]->has_half && dh[b + 1]->has_half &&
        wgs + (int64_t)dh[b + 1]->dp.Jw * dh[b + 1]->dp.S > cap &&
        (int64_t)dh[b]->dph.Jw * dh[b]->dph.S + (int64_t)dh[b + 1]->dph.Jw * dh[b + 1]->dph.S <= cap) {
      const lr_status st = run_decode(dh + b, dy + b, 2, X, M, stream, false, true);
      if (st == LR_OK) {
        b += 2;
        continue;
      }
      // refused before launching (the pair cannot be resident at once): run
      // them apart
      if (st != LR_ERR_UNSUPPORTED) return st;
    }
    int e = b + 1;
    while (e < nd && dh[e]->dp.kind == dh[b]->dp.kind && dh[e]->dp.kind < 2 && wgs + (int64_t)dh[e]->dp.Jw * dh[e]->dp.S <= cap) {
      wgs += (int64_t)dh[e]->dp.Jw * dh[e]->dp.S;
      ++e;
    }
    const lr_status st = run_decode(dh + b, dy + b, e - b, X, M, stream);
    if (st != LR_OK) return st;
    b = e;
  }
  if (np > 0) return run_prefill(ph, py, np, X, M, stream);
  return LR_OK;
}

// ------------------------------------------------- allocation-free decode ---
// lr_decode_noalloc keeps the in-place decode kernels' exchange tables in
// this file-scope device array instead of a handle's workspace.  Each GPU
// the library runs on holds its own copy until the process ends.  Host code
// never uses the array's name as an address: its device address is taken
// once per device with hipGetSymbolAddress and cached in g_scratch_ptr.
constexpr size_t kNoAllocScratchBytes = (size_t)64 << 20;
static __device__ __align__(256) unsigned char scratch[kNoAllocScratchBytes];
constexpr int kMaxDevices = 64;
std::mutex g_scratch_mu;
void* g_scratch_ptr[kMaxDevices];

// Device address of `scratch` on `dev` (nullptr and an error on failure).
lr_status scratch_address(int dev, void** out) {
  if (dev < 0 || dev >= kMaxDevices) return fail(LR_ERR_UNSUPPORTED, "device %d: at most %d devices", dev, kMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (!g_scratch_ptr[dev]) {
    void* p = nullptr;
    const hipError_t e = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
    if (e != hipSuccess || !p) return hip_fail(e != hipSuccess ? e : hipErrorInvalidSymbol, "hipGetSymbolAddress(scratch)");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return LR_OK;
}

// Zeroes n 16-byte words (a kernel rather than hipMemsetAsync, so that the
// clear is an ordinary kernel node when the caller captures a graph).
__global__ void clear_words_kernel(uint4* p, int n) {
  for (int i = blockIdx.x * blockDim.x + threadIdx.x; i < n; i += gridDim.x * blockDim.x) p[i] = make_uint4(0u, 0u, 0u, 0u);
}

}  // namespace

extern "C" {

const char* lr_status_str(lr_status s) {
  switch (s) {
    case LR_OK: return "LR_OK";
    case LR_ERR_INVALID_ARG: return "LR_ERR_INVALID_ARG";
    case LR_ERR_UNSUPPORTED: return "LR_ERR_UNSUPPORTED";
    case LR_ERR_OUT_OF_MEMORY: return "LR_ERR_OUT_OF_MEMORY";
    case LR_ERR_HIP: return "LR_ERR_HIP";
  }
  return "LR_ERR_UNKNOWN";
}

const char* lr_last_error(void) { return g_err; }

lr_status lr_linear_create(lr_linear** out, int64_t K, int64_t r, int64_t N, const void* A, const void* B,
                           int64_t max_M, uint32_t flags) {
  if (!out) return fail(LR_ERR_INVALID_ARG, "out must be non-null");
  *out = nullptr;
  lr_status st = lrv::check_create(K, r, N, A, B, max_M, flags, g_err, sizeof g_err);
  if (st != LR_OK) return st;

  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  hipDeviceProp_t prop;
  e = hipGetDeviceProperties(&prop, dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDeviceProperties");
  if (strncmp(prop.gcnArchName, "gfx950", 6) != 0)
    return fail(LR_ERR_UNSUPPORTED, "device %d is %s; these kernels are built for gfx950", dev, prop.gcnArchName);

  lr_linear* h = new (std::nothrow) lr_linear;
  if (!h) return fail(LR_ERR_OUT_OF_MEMORY, "host allocation failed");
  memset((void*)h, 0, sizeof *h);
  for (auto& ph : h->last_plan)
    for (auto& v : ph) v.store(-1);
  h->K = K;
  h->r = r;
  h->N = N;
  h->max_M = max_M;
  h->r_pad = lrv::round_up(r, 32);
  h->flags = flags;
  h->device = dev;
  h->A = (const uint16_t*)A;
  h->B = (const uint16_t*)B;

  h->has_decode = !(flags & LR_FLAG_FORCE_PREFILL) && max_M >= 1;
  h->has_prefill = !(flags & LR_FLAG_FORCE_DECODE) && (max_M > LR_DECODE_MAX_M || (flags & LR_FLAG_FORCE_PREFILL));
  h->dense = lrv::choose_dense(K, r, N, flags);

  size_t off = 0;
  size_t o_ctrl = 0, o_tcnt = 0, o_tflag = 0, o_ycnt = 0, o_tpart = 0, o_tfin = 0, o_ypart = 0, o_tbuf = 0;
  size_t o_sflags = 0, o_tsp = 0, o_asw = 0, o_bsw = 0, o_fpart = 0, o_pflags = 0;
  if (h->has_decode) h->dec_max_M = (int)(max_M < LR_DECODE_MAX_M ? max_M : LR_DECODE_MAX_M);
  h->stall_xor = (flags & LR_FLAG_TEST_STALL) ? lrk::kStallXor : 0u;
  h->spin_limit = (flags & LR_FLAG_TEST_STALL) ? 2048u : (1u << 22);
  if (h->has_decode && !h->dense && (flags & LR_FLAG_DECODE_XCD)) {
    // the XCD-sliced kernel: one workgroup per compute unit, all resident at
    // once (its workgroups wait on one another), so the occupancy of its
    // largest plan must allow at least one per compute unit
    const int cus = num_cus(dev);
    if (cus >= 8 && cus % 8 == 0) {
      h->xcd_P = cus / 8;
      int64_t lds = 0;
      for (int v = 0; v < 3; ++v) {
        const int pn = h->xcd_P >> v;
        h->xcd_ok[v] = pn >= 1 && (pn << v) == h->xcd_P && lrv::xcd_plan(K, r, N, pn, h->dec_max_M, &h->xp[v]);
        if (h->xcd_ok[v]) lds = lds > h->xp[v].lds ? lds : h->xp[v].lds;
      }
      if (h->xcd_ok[0] && lrk::decode_xcd_blocks_per_cu((int)lds) >= 1) h->dp.kind = 5;
    }
  }
  if (h->has_decode && !h->dense && h->dp.kind != 5) {
    const int occ = lrk::decode_blocks_per_cu();
    if (occ < 1) {
      delete h;
      return fail(LR_ERR_HIP, "decode kernel cannot be resident on this device");
    }
    h->dp = lrv::decode_partition(K, r, N, num_cus(dev),
                                  !(flags & LR_FLAG_DECODE_STREAMING) && lrk::decode_res_available(),
                                  (flags & LR_FLAG_DECODE_SPLIT) != 0, h->dec_max_M);
  }
  size_t o_xtf = 0, o_xyf = 0, o_xtp = 0, o_xyp = 0;
  if (h->has_decode && !h->dense && h->dp.kind == 5) {
    // XCD-sliced kernel: control words, one T and one Y flag per workgroup,
    // and the partial T and partial Y tables of the largest plan
    int64_t tp = 0, tf = 0, yp = 0;
    for (int v = 0; v < 3; ++v)
      if (h->xcd_ok[v]) {
        tp = tp > h->xp[v].tpart_bytes ? tp : h->xp[v].tpart_bytes;
        tf = tf > h->xp[v].tfin_bytes ? tf : h->xp[v].tfin_bytes;
        yp = yp > h->xp[v].ypart_bytes ? yp : h->xp[v].ypart_bytes;
      }
    o_ctrl = off;
    off = align_up(off + 64);
    o_xtf = off;
    off = align_up(off + (size_t)3 * 8 * h->xcd_P * 4);
    o_xtp = off;
    off = align_up(off + (size_t)tp);
    o_xyf = off;  // T of each XCD's range
    off = align_up(off + (size_t)tf);
    o_xyp = off;
    off = align_up(off + (size_t)yp);
    if (off >= ((size_t)1 << 31)) {
      delete h;
      return fail(LR_ERR_UNSUPPORTED, "decode workspace of %zu bytes exceeds 2 GiB", off);
    }
    h->dws_bytes = (int64_t)off;
  } else if (h->has_decode && !h->dense && (h->dp.kind >= 2)) {
    // role-split kernels: control words, replicated T slice flags and T
    // (the Y producers' reads of T spread over the replicas), and both
    // factors in the operand block layout
    const int readers = h->dp.kind >= 3 ? h->dp.g : h->dp.gb;
    h->nrep = readers < kSplitReplicas ? readers : kSplitReplicas;
    h->ldf = (int)lrv::round_up(h->dp.ga, 32);
    o_ctrl = off;
    off = align_up(off + 64);
    o_sflags = off;
    off = align_up(off + (size_t)h->nrep * h->ldf * 4);
    o_tsp = off;
    off = align_up(off + (size_t)h->nrep * (h->dec_max_M > 8 ? 2 : 1) * 16 * (32 * lrv::ceil_div(r, 32) + 8) * 2);
    if (h->dp.kind == 4) {
      o_fpart = off;
      off = align_up(off + (size_t)h->dp.ga * h->dp.maxc * 1024);
      o_pflags = off;
      off = align_up(off + (size_t)h->dp.ga * h->dp.maxc * 4);
    }
    o_asw = off;
    off = align_up(off + (size_t)h->dp.ga * lrv::ceil_div(K, 32) * 1024);
    o_bsw = off;
    off = align_up(off + (size_t)h->dp.gn * lrv::ceil_div(r, 32) * 1024);
    h->dws_bytes = (int64_t)off;
  } else if (h->has_decode && !h->dense) {
    const InplaceLayout L = inplace_layout(h->dp, h->dec_max_M, off);
    o_ctrl = L.ctrl;
    o_tcnt = L.tcnt;
    o_tflag = L.tflag;
    h->off_yflag = (uint32_t)L.yflag;
    o_ycnt = L.ycnt;
    o_tpart = L.tpart;
    o_tfin = L.tfin;
    o_ypart = L.ypart;
    off = L.end;
    h->has_half = false;
    if (h->dp.kind == 0) {
      // the half-machine plan's tables, laid out from the same start (same
      // control words; the epoch tags keep the two plans' words apart)
      h->dph = lrv::decode_streaming_partition(K, r, N, num_cus(dev) / 2);
      const InplaceLayout Lh = inplace_layout(h->dph, h->dec_max_M, L.ctrl);
      h->has_half = (int64_t)h->dph.Jw * h->dph.S <= num_cus(dev) / 2;
      h->hoff_tpart = (uint32_t)Lh.tpart;
      h->hoff_ypart = (uint32_t)Lh.ypart;
      if (h->has_half && Lh.end > off) off = Lh.end;
    }
    // resident kernel: its T exchange runs through one XCD's L2, so every
    // rank-slice group must sit on one XCD (Jw a multiple of 8); streaming
    // kernel: only a traffic-saving placement of adjacent rank slices
    h->xcd_local = (h->dp.kind == 1 ? h->dp.Jw % 8 == 0 : true) && xcd_map_ok(dev);
    if (off >= ((size_t)1 << 31)) {
      delete h;
      return fail(LR_ERR_UNSUPPORTED, "decode workspace of %zu bytes exceeds 2 GiB", off);
    }
    h->dws_bytes = (int64_t)off;
  }
  // the prefill kernels also form W for the dense fallback
  if ((h->has_prefill || (h->dense && h->has_decode)) && !lrk::prefill_available()) {
    delete h;
    return fail(LR_ERR_UNSUPPORTED, "device %d cannot give a workgroup %d bytes of LDS (prefill kernel)", dev,
                lrk::kPreLdsBytes);
  }
  size_t o_part = 0, o_w = 0, o_wsw = 0;
  if (h->has_prefill) {
    if (!h->dense) {
      o_tbuf = off;
      off = align_up(off + (size_t)max_M * h->r_pad * 2);
    }
    h->part_bytes = lrv::prefill_partial_bytes(max_M, K, h->r_pad, N, num_cus(dev), h->dense);
    o_part = off;
    off = align_up(off + (size_t)h->part_bytes);
  }
  if (h->dense && h->has_prefill) {
    o_w = off;
    off = align_up(off + (size_t)K * N * 2);
  }
  size_t o_dpart = 0, o_dcnt = 0;
  if (h->dense && h->has_decode) {
    o_wsw = off;
    off = align_up(off + (size_t)lrv::ceil_div(N, 16) * lrv::ceil_div(K, 32) * 1024);
    o_dpart = off;
    off = align_up(off + (size_t)lrk::kDenseMaxSplits * lrv::ceil_div(N, 16) * 1024);
    o_dcnt = off;
    off = align_up(off + (size_t)lrv::ceil_div(N, 16) * 4);
  }
  h->ws_bytes = off;
  if (off > 0) {
    e = hipMalloc(&h->ws, off);
    if (e != hipSuccess) {
      delete h;
      (void)hipGetLastError();
      return fail(LR_ERR_OUT_OF_MEMORY, "workspace hipMalloc(%zu): %s", off, hipGetErrorString(e));
    }
    e = hipMemset(h->ws, 0, off);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      (void)hipFree(h->ws);
      delete h;
      return hip_fail(e, "workspace clear");
    }
  }
  char* base = (char*)h->ws;
  if (h->has_decode && !h->dense) {
    // pinned host word for the decode kernels' timeout report
    e = hipHostMalloc((void**)&h->err_host, 64, hipHostMallocMapped | hipHostMallocCoherent);
    if (e == hipSuccess) {
      *h->err_host = 0u;
      e = hipHostGetDevicePointer((void**)&h->err_dev, h->err_host, 0);
    }
    if (e != hipSuccess) {
      (void)hipGetLastError();
      discard(h);
      return hip_fail(e, "pinned status word");
    }
  }
  if (h->has_decode && !h->dense && h->dp.kind == 5) {
    h->dws = base;
    h->ctrl = (uint32_t*)(base + o_ctrl);
    h->xflags = (uint32_t*)(base + o_xtf);
    h->xtpart = (float*)(base + o_xtp);
    h->xtfin = (float*)(base + o_xyf);
    h->xypart = (float*)(base + o_xyp);
    h->xcd_local = xcd_map_ok(dev);
  } else if (h->has_decode && !h->dense && (h->dp.kind >= 2)) {
    h->dws = base;
    h->ctrl = (uint32_t*)(base + o_ctrl);
    h->sflags = (uint32_t*)(base + o_sflags);
    h->Tsp = (uint16_t*)(base + o_tsp);
    h->fpart = h->dp.kind == 4 ? (float*)(base + o_fpart) : nullptr;
    h->pflags = h->dp.kind == 4 ? (uint32_t*)(base + o_pflags) : nullptr;
    h->Asw = (uint16_t*)(base + o_asw);
    h->Bsw = (uint16_t*)(base + o_bsw);
    e = lrk::launch_dense_swizzle(h->A, h->Asw, K, r, nullptr);
    if (e == hipSuccess) e = lrk::launch_dense_swizzle(h->B, h->Bsw, r, N, nullptr);
    if (e == hipSuccess) e = hipDeviceSynchronize();
    if (e != hipSuccess) {
      discard(h);
      return hip_fail(e, "split decode: factor layout");
    }
  } else if (h->has_decode && !h->dense) {
    h->dws = base;  // the decode regions start the workspace
    h->ctrl = (uint32_t*)(base + o_ctrl);
    h->tcnt = (uint32_t*)(base + o_tcnt);
    h->tflag = (uint32_t*)(base + o_tflag);
    h->ycnt = (uint32_t*)(base + o_ycnt);
    h->off_tpart = (uint32_t)o_tpart;
    h->off_tfin = (uint32_t)o_tfin;
    h->off_ypart = (uint32_t)o_ypart;
    h->off_tflag = (uint32_t)o_tflag;
  }
  if (h->has_decode && !h->dense) {
    // The decode kernels' workgroups wait on one another, so a launch
    // completes only if all of them are resident at once: every launch this
    // handle makes alone is checked against the occupancy of its kernel
    // (M = 1 and the largest M select different variants), with nothing
    // launched.  The pointers below are never dereferenced.
    static uint16_t probe;
    const lr_linear* self = h;
    uint16_t* yprobe = &probe;
    const int64_t ms[2] = {1, h->dec_max_M};
    for (int64_t m : ms) {
      const lr_status cst = run_decode(&self, &yprobe, 1, &probe, m, nullptr, true);
      if (cst != LR_OK) {
        discard(h);
        return cst;
      }
    }
  }
  if (h->has_prefill) {
    h->Tbuf = h->dense ? nullptr : (uint16_t*)(base + o_tbuf);
    h->part = h->part_bytes > 0 ? (float*)(base + o_part) : nullptr;
  }
  if (h->dense && (h->has_decode || h->has_prefill)) {
    // W lives in the workspace when prefill reads it; a decode-only handle
    // keeps just the decode layout and forms W in a temporary buffer
    void* tmp = nullptr;
    if (h->has_prefill) {
      h->W = (uint16_t*)(base + o_w);
    } else {
      e = hipMalloc(&tmp, (size_t)K * N * 2);
      if (e != hipSuccess) {
        (void)hipGetLastError();
        discard(h);
        return fail(LR_ERR_OUT_OF_MEMORY, "dense fallback: hipMalloc(%lld) for W", (long long)(K * N * 2));
      }
    }
    if (h->has_decode) {
      h->Wsw = (uint16_t*)(base + o_wsw);
      h->dpart = (float*)(base + o_dpart);
      h->dcnt = (uint32_t*)(base + o_dcnt);
    }
    st = form_dense(h, h->W ? h->W : (uint16_t*)tmp);
    if (tmp) (void)hipFree(tmp);
    if (st != LR_OK) {
      discard(h);
      return st;
    }
  }
  *out = h;
  return LR_OK;
}

lr_status lr_linear_run(const lr_linear* h, const void* X, void* Y, int64_t M, void* stream) {
  if (!h) return fail(LR_ERR_INVALID_ARG, "handle is null");
  lrv::Shape s{h->K, h->r, h->N, h->max_M, h->A, h->B};
  lr_status st = lrv::check_run(s, X, Y, M, g_err, sizeof g_err);
  if (st != LR_OK) return st;
  st = take_stall(h);
  if (st != LR_OK || M == 0) return st;
  uint16_t* Ys[1] = {(uint16_t*)Y};
  const lr_linear* hs[1] = {h};
  if (use_decode(h, M) && h->dense) return run_dense_decode(hs, Ys, 1, X, M, (hipStream_t)stream);
  if (use_decode(h, M)) return run_decode(hs, Ys, 1, X, M, (hipStream_t)stream);
  return run_prefill(hs, Ys, 1, X, M, (hipStream_t)stream);
}

lr_status lr_decode_noalloc(const void* X, const void* A, const void* B, void* Y, int64_t M, int64_t K, int64_t r,
                            int64_t N, uint32_t* status, void* stream) {
  lr_status st = lrv::check_create(K, r, N, A, B, M, LR_FLAG_FACTORED, g_err, sizeof g_err);
  if (st != LR_OK) return st;
  if (M > LR_DECODE_MAX_M) return fail(LR_ERR_INVALID_ARG, "M=%lld: this entry point takes M <= %d", (long long)M, LR_DECODE_MAX_M);
  lrv::Shape s{K, r, N, M, A, B};
  st = lrv::check_run(s, X, Y, M, g_err, sizeof g_err);
  if (st != LR_OK || M == 0) return st;
  if (status && reinterpret_cast<uintptr_t>(status) % 4 != 0) return fail(LR_ERR_INVALID_ARG, "status must be 4-byte aligned");
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return hip_fail(e, "hipGetDevice");
  // the plan lr_linear_create makes by default for max_M = M, on a handle
  // that lives on this stack frame and points into the scratch array
  lr_linear h{};
  h.K = K;
  h.r = r;
  h.N = N;
  h.max_M = M;
  h.flags = LR_FLAG_FORCE_DECODE | LR_FLAG_FACTORED;
  h.device = dev;
  h.A = (const uint16_t*)A;
  h.B = (const uint16_t*)B;
  h.has_decode = true;
  h.dec_max_M = (int)M;
  h.dp = lrv::decode_partition(K, r, N, num_cus(dev), lrk::decode_res_available(), false, M);
  if (h.dp.kind != 0 && h.dp.kind != 1) return fail(LR_ERR_UNSUPPORTED, "no in-place decode plan for this shape");
  const InplaceLayout L = inplace_layout(h.dp, (int)M, 0);
  if (L.end > kNoAllocScratchBytes)
    return fail(LR_ERR_UNSUPPORTED, "this shape needs %zu bytes of decode scratch; the allocation-free entry point has %zu",
                L.end, kNoAllocScratchBytes);
  void* base = nullptr;
  st = scratch_address(dev, &base);
  if (st != LR_OK) return st;
  char* b = (char*)base;
  h.dws = b;
  h.dws_bytes = (int64_t)L.end;
  h.ctrl = (uint32_t*)(b + L.ctrl);
  h.tcnt = (uint32_t*)(b + L.tcnt);
  h.tflag = (uint32_t*)(b + L.tflag);
  h.ycnt = (uint32_t*)(b + L.ycnt);
  h.off_tpart = (uint32_t)L.tpart;
  h.off_tfin = (uint32_t)L.tfin;
  h.off_ypart = (uint32_t)L.ypart;
  h.off_tflag = (uint32_t)L.tflag;
  h.off_yflag = (uint32_t)L.yflag;
  h.xcd_local = false;  // the placement check would allocate: exchange device-coherent
  h.spin_limit = 1u << 22;
  h.stall_xor = 0u;
  h.err_dev = status;
  // The array keeps the last call's contents, which may be another shape's
  // tables: the control words (generation, counters, flags) start at zero
  // every call, and so do the epoch-tagged exchange words, so no stale flag
  // or tag can match this call's epoch.
  const int vecs = (int)(L.end / 16);  // the layout's regions are 256-byte aligned
  const int clear_blocks = (vecs + 255) / 256 < 1024 ? (vecs + 255) / 256 : 1024;
  hipLaunchKernelGGL(clear_words_kernel, dim3((unsigned)clear_blocks), dim3(256), 0, (hipStream_t)stream,
                     reinterpret_cast<uint4*>(b), vecs);
  e = hipGetLastError();
  if (e != hipSuccess) return hip_fail(e, "scratch clear launch");
  const lr_linear* hs[1] = {&h};
  uint16_t* Ys[1] = {(uint16_t*)Y};
  return run_decode(hs, Ys, 1, X, M, (hipStream_t)stream);
}

lr_status lr_group_run(const lr_linear* const* hs, int n, const void* X, void* const* Ys, int64_t M, void* stream) {
  if (!hs || !Ys) return fail(LR_ERR_INVALID_ARG, "handle and output arrays must be non-null");
  if (n < 1 || n > lrv::kMaxGroup) return fail(LR_ERR_INVALID_ARG, "n=%d projections; 1 to %d share X", n, lrv::kMaxGroup);
  lrv::Shape s[lrv::kMaxGroup];
  const void* yv[lrv::kMaxGroup];
  uint16_t* ys[lrv::kMaxGroup];
  for (int i = 0; i < n; ++i) {
    if (!hs[i]) return fail(LR_ERR_INVALID_ARG, "handle %d is null", i);
    for (int j = 0; j < i; ++j)
      if (hs[j] == hs[i])
        return fail(LR_ERR_INVALID_ARG, "handles %d and %d are the same (each owns a workspace)", j, i);
    s[i] = lrv::Shape{hs[i]->K, hs[i]->r, hs[i]->N, hs[i]->max_M, hs[i]->A, hs[i]->B};
    yv[i] = Ys[i];
    ys[i] = (uint16_t*)Ys[i];
  }
  lr_status st = lrv::check_group(s, n, X, yv, M, g_err, sizeof g_err);
  if (st != LR_OK) return st;
  for (int i = 0; i < n; ++i) {
    const lr_status si = take_stall(hs[i]);
    if (si != LR_OK) st = si;
  }
  if (st != LR_OK || M == 0) return st;
  return run_group(hs, ys, n, X, M, (hipStream_t)stream);
}

lr_status lr_mlp_packed_run(const lr_linear* gate, const lr_linear* up, const void* X, void* Y_gate, void* Y_up,
                            int64_t M, void* stream) {
  if (!gate || !up) return fail(LR_ERR_INVALID_ARG, "gate and up handles must be non-null");
  const lr_linear* hs[2] = {gate, up};
  void* Ys[2] = {Y_gate, Y_up};
  return lr_group_run(hs, 2, X, Ys, M, stream);
}

void lr_linear_destroy(lr_linear* h) {
  if (!h) return;
  if (h->ws || h->err_host) {
    // A handle may be released (e.g. by a garbage collector) while another
    // stream captures a graph.  hipFree and hipHostFree are not allowed
    // under a global-mode capture and would invalidate it; in relaxed mode
    // this thread's frees leave other captures alone.  (The caller must not
    // free a handle that a graph being captured or replayed still uses.)
    hipStreamCaptureMode mode = hipStreamCaptureModeRelaxed;
    const bool swapped = hipThreadExchangeStreamCaptureMode(&mode) == hipSuccess;
    if (h->ws) (void)hipFree(h->ws);
    if (h->err_host) (void)hipHostFree(h->err_host);
    if (swapped) (void)hipThreadExchangeStreamCaptureMode(&mode);
  }
  delete h;
}

lr_status lr_linear_status(const lr_linear* h) {
  if (!h) return fail(LR_ERR_INVALID_ARG, "handle is null");
  return take_stall(h);
}

lr_status lr_linear_describe(const lr_linear* h, char* buf, int64_t len) {
  if (!h || !buf || len <= 0) return fail(LR_ERR_INVALID_ARG, "null handle or buffer");
  char dec[200];
  if (h->dp.kind == 5)
    snprintf(dec, sizeof dec, "kind=xcd P=%d pa=%d rs=%d nc=%d cpr_a=%d cpr_b=%d da=%d db=%d lds=%lld grid=%d",
             h->xcd_P, h->xp[0].pa, h->xp[0].rs, h->xp[0].nc, h->xp[0].cpr_a, h->xp[0].cpr_b, h->xp[0].da,
             h->xp[0].db, (long long)h->xp[0].lds, 8 * h->xcd_P);
  else if (h->dp.kind == 2)
    snprintf(dec, sizeof dec, "kind=split GA=%d GB=%d gpw=%d blocks_per_wave=%d grid=%d", h->dp.ga, h->dp.gb,
             h->dp.gpw, h->dp.ntps, h->dp.ga + h->dp.gb);
  else if (h->dp.kind == 3)
    snprintf(dec, sizeof dec, "kind=split_stream GA=%d GY=%d nt=%d blocks_per_wave=%d grid=%d", h->dp.ga, h->dp.gb,
             h->dp.nt, h->dp.ntps, h->dp.g);
  else if (h->dp.kind == 4)
    snprintf(dec, sizeof dec, "kind=split_flat GA=%d maxc=%d blocks_per_wave=%d grid=%d", h->dp.ga, h->dp.maxc,
             h->dp.ntps, h->dp.g);
  else
    snprintf(dec, sizeof dec, "kind=%s Jw=%d JS=%d S=%d ktps=%d ntps=%d grid=%d",
             h->dp.kind == 1 ? "resident" : "streaming", h->dp.Jw, h->dp.js_w, h->dp.S, h->dp.ktps, h->dp.ntps,
             h->dp.Jw * h->dp.S);
  snprintf(buf, (size_t)len,
           "K=%lld r=%lld N=%lld r_pad=%lld max_M=%lld dense=%d decode=%d[%s] "
           "xcd_local=%d prefill=%d[last phase1 kind=%d nb=%d splits=%d, phase2 kind=%d nb=%d splits=%d] "
           "workspace=%zu",
           (long long)h->K, (long long)h->r, (long long)h->N, (long long)h->r_pad, (long long)h->max_M,
           (int)h->dense, (int)h->has_decode, dec, (int)h->xcd_local, (int)h->has_prefill,
           h->last_plan[0][0].load(), h->last_plan[0][1].load(), h->last_plan[0][2].load(), h->last_plan[1][0].load(),
           h->last_plan[1][1].load(), h->last_plan[1][2].load(), h->ws_bytes);
  return LR_OK;
}

int64_t lr_linear_workspace_bytes(const lr_linear* h) { return h ? (int64_t)h->ws_bytes : 0; }

#ifdef LR_DECODE_TRACE
// Trace builds only: device buffer of grid * 8 uint64 phase timestamps.
void lr_debug_set_trace(void* device_buf) { g_trace = (uint64_t*)device_buf; }
void lr_debug_set_xcd_coherent(int on) { g_xcd_coherent = on != 0; }
#endif

}  // extern "C"
