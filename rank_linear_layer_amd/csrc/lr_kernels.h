// Internal interface between the C-ABI host library and the HIP kernels.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <atomic>

namespace lrk {

// Raise a kernel's dynamic-LDS limit to `bytes` once per device (the limit
// is a property of the kernel on the current device; `done` holds one bit
// per device id below 64, set after a successful call, so concurrent first
// calls at worst set it twice).
inline hipError_t ensure_dynamic_lds(const void* kernel, int bytes, std::atomic<uint64_t>& done) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t bit = dev >= 0 && dev < 64 ? (uint64_t)1 << dev : 0;
  if (bit && (done.load(std::memory_order_acquire) & bit)) return hipSuccess;
  e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
  if (e == hipSuccess && bit) done.fetch_or(bit, std::memory_order_release);
  return e;
}

// Kernels whose workgroups wait on one another complete only when every
// workgroup of the grid is resident at once.  True when `grid` workgroups of
// `kernel` (`threads` each, `lds` bytes of dynamic LDS) fit the current
// device together: the occupancy calculator's workgroups per compute unit
// times the compute units.  The last answer is cached per kernel instance
// in `cache` (device, LDS bytes, capacity), so a launch pays for the query
// only when one of them changes.
inline hipError_t check_coresident(const void* kernel, int threads, size_t lds, int64_t grid,
                                   std::atomic<uint64_t>& cache) {
  int dev = 0;
  hipError_t e = hipGetDevice(&dev);
  if (e != hipSuccess) return e;
  const uint64_t key = ((uint64_t)(dev & 0xFF) << 56) | ((uint64_t)(lds & 0xFFFFFF) << 32);
  uint64_t c = cache.load(std::memory_order_acquire);
  if ((c & 0x80000000u) == 0 || (c & ~(uint64_t)0xFFFFFFFFu) != key) {
    int per_cu = 0, cus = 0;
    e = hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, threads, lds);
    if (e != hipSuccess) return e;
    e = hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
    if (e != hipSuccess) return e;
    const int64_t cap = (int64_t)per_cu * cus;
    c = key | 0x80000000u | (uint64_t)(cap < 0x7FFFFFFF ? cap : 0x7FFFFFFF);
    cache.store(c, std::memory_order_release);
  }
  return grid <= (int64_t)(c & 0x7FFFFFFFu) ? hipSuccess : hipErrorCooperativeLaunchTooLarge;
}

// Bounded waits.  Every cross-workgroup wait of the decode kernels gives up
// after `spin_limit` polls; it then raises the handle's device word ctrl[2]
// and stores 1 to `err`, a word of pinned host memory that the host library
// reads before the handle's next call.  `stall_xor` is XORed into the flag
// value the T hand-off waits for: zero in normal use; a test sets its top
// bit, so that this wait can never succeed and must give up while every
// workgroup still runs to its end.
constexpr uint32_t kStallXor = 0x80000000u;

// ---------------------------------------------------------------- decode ---
// Tile geometry of the fused decode kernel (M <= 16).
constexpr int kDecThreads = 256;  // 4 waves
constexpr int kDecWaves = 4;
constexpr int kDecJS = 120;       // rank columns per j-slice (15 producing lanes x 8)
constexpr int kDecKT = 32;        // K rows per k-tile (one MFMA K-step)
constexpr int kDecNT = 120;       // output columns per n-tile
constexpr int kDecMaxProj = 4;    // projections sharing X in one launch

// One factorized projection inside a decode launch.  The launch's
// workgroups [wg_begin, wg_begin + Jw*S) belong to it; workgroup
// (js, s) = (local / S, local % S) computes the partial T of rank slice js
// over K slice s, then the partial Y of rank slice js over N slice s.
// Workspace regions are byte offsets from `ws` (one buffer resource):
//   off_tpart  [Jw*S][M][kDecJS] fp32   GEMM1 partials
//   off_tfin   [Jw][M][kDecJS]   fp32   reduced T slices
//   off_ypart  [S][Jw][ntps][M][kDecNT] fp32 GEMM2 partials (resident kernel:
//              each value beside a 32-bit epoch tag, twice the bytes)
struct DecProj {
  const uint16_t* A;
  const uint16_t* B;
  uint16_t* Y;
  const void* ws;
  uint32_t* ctrl;   // [0] generation (launch stamp - 1), [1] finished n-slices, [2] spin-timeout flag
  uint32_t* tcnt;   // [Jw] arrivals of T partials (self-resetting)
  uint32_t* tflag;  // epoch stamps: [Jw] published T slices (streaming), [Jw*S] partials (resident)
  uint32_t* ycnt;   // [S] arrivals of Y partials (self-resetting)
  int64_t ws_bytes;
  uint32_t off_tpart, off_tfin, off_ypart;
  uint32_t off_tflag, off_yflag;  // resident kernel: [Jw*S] flag words each
  int r, N, Jw, S, ktps, ntps, wg_begin;
  int js_w;       // rank columns per slice
  int xcd_local;  // workgroups are dealt to XCDs round-robin (verified) and wg_begin % 8 == 0:
                  // resident kernel: rank-slice groups share an XCD; streaming: adjacent slices do
  uint32_t* err;  // pinned host word set to 1 when a wait gives up (null: none)
  uint32_t spin_limit, stall_xor;
};

struct DecArgs {
  const uint16_t* X;
  uint64_t* trace;  // per-workgroup phase timestamps (builds with LR_DECODE_TRACE only)
  int M, K, nproj;
  int check_only;   // the launcher validates and checks residency, and launches nothing
  DecProj p[kDecMaxProj];
};
constexpr int kDecTracePoints = 16;

hipError_t launch_decode(const DecArgs& args, int grid, hipStream_t stream);

// LDS-resident decode kernel (lr_decode_res.hip): 128-column rank slices,
// every slab of a workgroup held in LDS at once.
constexpr int kResThreads = 256;
constexpr int kResJS = 128;
constexpr int kResKT = 32;
constexpr int kResNT = 128;
constexpr int kResMaxKt = 8;   // k-tiles per workgroup
constexpr int kResMaxNt = 2;   // n-tiles per workgroup
constexpr int kResCA = kResJS / 8 + 1;                 // chunks per A row run
constexpr int kResXK = kResMaxKt * kResKT;             // X columns staged
constexpr int kResXBytes = 16 * kResXK * 2;
constexpr int kResABytes = kResMaxKt * kResKT * kResCA * 16;
constexpr int kResBBytes = kResJS * (kResNT / 8 * kResMaxNt + 1) * 16;
constexpr int kResRedBytes = 4 * 16 * kResJS * 4;
constexpr int kResLdsBytes = kResXBytes + kResABytes + kResBBytes;
static_assert(kResRedBytes + 16 * (kResJS + 8) * 4 <= kResABytes, "reduction buffers must fit the A region");
hipError_t launch_decode_res(const DecArgs& args, int grid, hipStream_t stream);
// True when the device accepts kResLdsBytes of LDS per workgroup.
bool decode_res_available();
// True when workgroup i of a `grid`-sized launch runs on XCD i % 8 for every i
// (checked with HW_REG_XCC_ID).
bool xcd_round_robin(int grid);
// Workgroups of the decode kernel that one compute unit holds at once (0 on error).
int decode_blocks_per_cu();

// Role-split decode kernel (lr_decode_split.hip): workgroups [0, GA) each
// produce 16 rank columns of T over all of K, workgroups [GA, GA + GB) each
// produce gpw 16-column groups of Y over the whole rank.  Asw and Bsw are A
// (K x r) and B (r x N) in the dense path's decode layout (see DenseArgs).
constexpr int kSplitMaxBlocks = 16;  // B blocks a wave of a Y producer holds
constexpr int64_t kSplitMaxTBytes = 144 * 1024;  // LDS for T's operand planes (whole KB) in a Y producer
struct SplitArgs {
  const uint16_t* X;    // [M x K] bf16
  const uint16_t* Asw;  // ceil(r/16) groups x nkA blocks
  const uint16_t* Bsw;  // ceil(N/16) groups x nkB blocks
  uint16_t* Y;          // [M x N] bf16
  uint16_t* P;          // nrep replicas of T as GEMM2 operand planes, each 16 x ldp bf16: with M <= 8
                        // one plane (rows 0-7 bf16 hi of T, rows 8-15 bf16 lo), else two (hi, lo of
                        // 16 rows); columns >= 16 GA stay zero
  uint32_t* flags;      // nrep replicas of [GA] epoch stamps of published T slices (replica stride ldf)
  uint32_t* ctrl;       // [0] generation, [1] Y producers past the T wait, [2] spin-timeout flag
  uint64_t* trace;      // per-workgroup phase timestamps (builds with LR_DECODE_TRACE only)
  int nrep, ldf;        // replicas of T and of the flags; flag words per replica (multiple of 32)
  int M, K, r, N;
  int nkA, nkB;         // ceil(K/32), ceil(r/32)
  int ldp;              // 32 nkB + 8 (plane rows staggered across LDS banks)
  int GA, GN, GB, gpw;  // T producers = ceil(r/16); column groups = ceil(N/16); Y producers; groups each
  // streaming variant (stream_y = 1): G workgroups, all computing Y; the
  // first GA produce T first and take nt column groups each, the other
  // G - GA share the rest.  Every wave keeps its T operands in registers.
  int stream_y, G, nt;
  // flat variant (stream_y = 2): every workgroup takes TB / G of A's blocks
  // in slice-major order (TB = GA nkA) and GN / G column groups of Y; the
  // first contributor of a slice adds the others' partials
  float* part;          // [GA][maxc] tiles of 16 x 16 fp32
  uint32_t* pflags;     // [GA][maxc] epoch stamps of the partial tiles
  int maxc;             // contributors per slice the table holds (>= ceil(nkA / max(1, TB / G)) + 1)
  uint32_t* err;        // pinned host word set to 1 when a wait gives up (null: none)
  uint32_t spin_limit, stall_xor;
  int check_only;       // the launcher validates and checks residency, and launches nothing
};
hipError_t launch_decode_split(const SplitArgs& args, hipStream_t stream);
// B blocks per wave of a Y producer for this plan (<= kSplitMaxBlocks to launch).
int split_blocks_per_wave(const SplitArgs& args);

// XCD-sliced decode kernel (lr_decode_xcd.hip): one workgroup per compute
// unit; XCD x owns rank rows [x r / 8, (x + 1) r / 8) of each projection,
// and projection p's workgroups are local indices [p0, p0 + pn) of every
// XCD (workgroup g runs on XCD g % 8, local index g / 8).  A and B are read
// in place.  Exchange tables hold fp32 columns of 4 mq rows (mq =
// ceil(M / 4)), column-major.
constexpr int kXcdMaxProj = 4;          // projections sharing X in one launch
constexpr int kXcdMaxLds = 160 * 1024;  // dynamic LDS limit of the kernel
constexpr int kXcdTilesA = 16;          // 16-column GEMM1 tiles per rank sub-range (256 columns)
constexpr int kXcdTilesB = 16;          // 16-column GEMM2 tiles per column chunk (256 columns)
struct XcdProj {
  const uint16_t* A;  // [K x r] bf16 row-major
  const uint16_t* B;  // [r x N]
  uint16_t* Y;        // [M x N]
  uint32_t* ctrl;     // [0] generation, [1] workgroups finished, [2] a wait timed out
  uint32_t* err;      // device address of the host-visible timeout word (may be null)
  uint32_t* flags;    // [3][8 pn] epoch stamps: partial T stored, T columns reduced, partial Y stored
  float* tpart;       // [8 (pa / rs)][ldtp][4 mq] partial T of each (XCD, K-slab) over the XCD's rank range
  float* tfin;        // [8][ldtp][4 mq] T of each XCD's rank range
  float* ypart;       // [8 (pn - pa)][ws][4 mq] partial Y of each B workgroup's column slab
  int r, N;
  int p0, pn;         // local workgroup indices [p0, p0 + pn) of this projection on every XCD
  int pa, rs;         // the first pa of them stream A: (pa / rs) K-slabs x rs rank sub-ranges;
                      // the other pn - pa stream B, one column slab each
  int nc;             // column chunks of a B slab (1, 2, 4 or 8; wave w takes chunk w % nc)
  int cpr_a, cpr_b;   // 16-byte chunks per LDS row of an A piece / of a B chunk (even)
  int da, db;         // k-steps in flight per wave of an A / a B workgroup
  int ldtp, ws;       // rank range (>= ceil(r/8)) and slab (>= ceil(N/(pn - pa))) lengths of the tables
  uint32_t stall_xor; // XORed into the value the partial-T wait expects (a test sets kStallXor)
};
struct XcdArgs {
  const uint16_t* X;  // [M x K] bf16
  int M, K;
  int nproj, grid;    // grid = 8 x (sum of pn)
  int xcd_local;      // 1: the T exchange runs through each XCD's L2 (workgroup placement verified)
  uint32_t spin_limit;
  uint64_t* trace;    // phase timestamps (builds with LR_DECODE_TRACE only)
  int check_only;     // the launcher validates and checks residency, and launches nothing
  XcdProj p[kXcdMaxProj];
};
hipError_t launch_decode_xcd(const XcdArgs& args, int lds_bytes, hipStream_t stream);
// Workgroups of the XCD-sliced kernel a compute unit holds at once with
// lds_bytes of dynamic LDS (0 on error).
int decode_xcd_blocks_per_cu(int lds_bytes);

// ----------------------------------------------------------------- dense ---
// Dense fallback (W = A . B precomputed).  Wsw is W in the decode layout:
// ceil(N/16) column groups x ceil(K/32) k-steps of 1 KB blocks, each block
// the 16x16x32 MFMA B operand of that group and step (zero past K and N).
constexpr int kDenseMaxOut = 4;  // projections sharing X in one dense decode launch
constexpr int kDenseMaxSplits = 16;  // K slices of one column group (workgroups that share it)
struct DenseOut {
  const uint16_t* Wsw;  // decode layout of this projection's W
  uint16_t* Y;          // [M x N] bf16
  int64_t N;
  float* part;          // [splits][ceil(N/16)][256] fp32 partial tiles (splits > 1)
  uint32_t* cnt;        // [ceil(N/16)] arrivals per column group, zero between launches
};
struct DenseArgs {
  const uint16_t* X;    // [M x K] bf16
  int64_t M, K;
  int64_t nk;           // ceil(K / 32)
  int64_t ng;           // column groups of all outputs
  int nout;             // 1 .. kDenseMaxOut outputs; workgroups are dealt output by output
  int splits;           // 1 .. kDenseMaxSplits K slices per column group
  int pad_;
  DenseOut o[kDenseMaxOut];
};
// Wsw from W (row-major [K x N]); Wsw holds ceil(N/16)*ceil(K/32)*512 bf16.
hipError_t launch_dense_swizzle(const uint16_t* W, uint16_t* Wsw, int64_t K, int64_t N, hipStream_t stream);
// Y_i = X . W_i for M <= 16: `splits` workgroups per 16-column group of
// every output, each over a slice of K; the last of a group's workgroups to
// finish adds the fp32 partials in slice order (nothing waits).
hipError_t launch_dense_decode(const DenseArgs& args, hipStream_t stream);

// --------------------------------------------------------------- prefill ---
constexpr int kPreMaxOut = 4;   // projections sharing X in one prefill launch
constexpr int kPreThreads = 512;  // 8 waves (two per SIMD)
constexpr int kPreBM = 256;       // rows per workgroup tile
constexpr int kPreKT = 32;        // k per LDS stage (one MFMA k-step)
// columns per workgroup tile = 32 * nb, nb in [kPreMinNB, kPreMaxNB]
constexpr int kPreMinNB = 2;
constexpr int kPreMaxNB = 7;
constexpr int kPreSlotBytes = (16 + 15) * 1024;  // one k-step: P (16 KB) + Q of the widest tile (15 KB)
constexpr int kPreSlots = 5;                      // ring of k-steps in LDS
constexpr int kPreLdsBytes = kPreSlots * kPreSlotBytes + 1024;  // + a spare 1 KB for loads that fill nothing

// C[rows x out_cols] = P[rows x kd] . Q[kd x ldq] for one or two column
// blocks in one launch.  P is k-contiguous (X or T); Q is row-major with
// leading dimension ldq (= its column count) and qrows valid rows (rows
// beyond qrows read as zero).  Output columns in [ldq, out_cols) are 0.
struct PreOut {
  const uint16_t* P;
  const uint16_t* Q;
  uint16_t* C;
  int64_t ldp;      // leading dimension of P
  int64_t kd;       // reduction length
  int64_t ldq;      // = valid columns of Q
  int64_t qrows;    // valid rows of Q
  int64_t ldc;      // leading dimension of C
  int64_t out_cols; // columns of C to write
  float* part;      // k-split fp32 partials [splits][rows][ldpart] (splits > 1)
  int64_t ldpart;   // >= out_cols, multiple of 4
  int col_tiles;    // column tiles of this block
  int pad_;
};
struct PreArgs {
  int64_t rows;     // M
  int nout;         // 1 .. kPreMaxOut column blocks (projections sharing P's rows)
  int row_tiles;
  int nb;           // MFMA column blocks per wave: the tile is 32 * nb columns wide
  int splits;       // k-splits per tile (1: the GEMM writes bf16 C itself)
  int split_steps;  // 32-deep k-steps per split
  int pad_;
  PreOut o[kPreMaxOut];
};
hipError_t launch_prefill_gemm(const PreArgs& args, hipStream_t stream);
// One wave per SIMD, 256 x 256 tiles, for a 16-byte aligned P (nb = 8, even
// split_steps, equal weight leading dimensions mod 8 across outputs).
hipError_t launch_prefill_w4(const PreArgs& args, hipStream_t stream);
// C[rows x cols] = bf16(sum of `splits` fp32 partials, in split order).
hipError_t launch_prefill_reduce(const float* part, int splits, int64_t rows, int64_t cols, int64_t ldpart,
                                 uint16_t* C, int64_t ldc, hipStream_t stream);
// True when the device accepts kPreLdsBytes of LDS per workgroup.
bool prefill_available();

}  // namespace lrk
