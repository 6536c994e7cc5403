// Prefill kernels (M > 16): LDS-staged MFMA GEMMs with on-chip rank padding.
//
// Prefill is compute-bound ("LowRankArena ...", "Why theoretical FLOPs
// saved does not equal faster inference": many tokens at once, arithmetic
// throughput is the bottleneck), so both products run on the bf16 matrix
// cores with fp32 accumulation:
//   phase 1  T[M x r_pad] = X . A      (T stored bf16 in the workspace;
//                                       columns r..r_pad-1 written as 0)
//   phase 2  Y[M x N]     = T . B      (reduction over r_pad; B rows >= r
//                                       read as 0, never fetched)
// The rank is padded to the 32-wide MFMA K-step on chip only; A and B keep
// their public shapes.  Any r mod 8 and N mod 8 is handled by the same
// kernel: misaligned weight rows are realigned in registers (see
// lr_device.h), misaligned output rows are written through an LDS staging
// tile that mirrors each row's alignment.
//
// Workgroup tile: 256 rows x 240 columns, 64-deep k-steps, 4 waves, one
// workgroup per compute unit.  Wave w owns rows [64w, 64w + 64) and all 240
// columns: 4 x 15 MFMA 16x16x32 tiles, 240 fp32 accumulators per lane.
//
// Per k-step the workgroup stages two operand tiles in LDS (double
// buffered, 2 x 63 KB):
//   P tile  256 rows x 64 k   (X or T; k-contiguous, copied as is)
//   Q tile  240 cols x 64 k   (A or B transposed: each lane loads 8 rows x
//                              8 columns, realigns and transposes them in
//                              registers, and writes 8 k-contiguous column
//                              segments)
// Both tiles use one layout, built from blocks of 16 rows (or columns) x 8
// chunks of 16 bytes: chunk c of line L of block b sits at
//   b * 2080 + 256 c + 16 sigma(L),   sigma(L) = ((L & 7) << 1) | (L >> 3).
// An MFMA operand read (16 consecutive lines, one chunk) and a transposing
// write (lines 8j + e for 16 lanes j) both touch 16 distinct 16-byte bank
// groups, and the operand address is one per-lane base plus a compile-time
// offset.  With an aligned P the P tile is filled by direct-to-LDS buffer
// loads (no registers), in the same layout.
//
// Grid: tiles are dealt so that each XCD (workgroup id mod 8) gets one
// contiguous run of the tile order, and the order walks groups of four row
// tiles column by column: the workgroups resident on one XCD share their P
// and Q panels in that XCD's L2.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

namespace {

constexpr int kBM = kPreBM;          // 256
constexpr int kBN = kPreBN;          // 240
constexpr int kBK = kPreKT;          // 64
constexpr int kBlk = 2080;           // one 16-line block: 16 x 8 chunks + 32 bytes of skew
constexpr int kStageQ = 15 * kBlk;   // Q tile bytes (240 columns)
constexpr int kStageP = 16 * kBlk;   // P tile bytes (256 rows)
constexpr int kStage = kStageQ + kStageP;
constexpr int kEpiRS = 496;          // epilogue staging row pitch (31 chunks)
constexpr int kGroupRows = 4;        // row tiles per group in the tile order
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;
static_assert(kPreLdsBytes == 2 * kStage, "LDS size");
static_assert(kBM * kEpiRS <= 2 * kStage, "epilogue staging must fit the stage buffers");

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ int sigma(int L) { return ((L & 7) << 1) | (L >> 3); }
__device__ __forceinline__ int sigma_inv(int s) { return ((s & 1) << 3) | (s >> 1); }

__device__ __forceinline__ u32x4_t lds_read16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

struct Tile {
  int bi;      // output block (0 or 1)
  int64_t mb;  // first row
  int64_t nb;  // first column
};

// Workgroup id -> tile.  XCD x (= id mod 8) receives the contiguous run
// [x*q + min(x, rem), ...) of the tile order; the order is row-tile groups of
// kGroupRows, walked column tile by column tile across both outputs.
__device__ __forceinline__ Tile map_tile(const PreArgs& a) {
  const int ct_total = a.o[0].col_tiles + (a.nout > 1 ? a.o[1].col_tiles : 0);
  const int total = a.row_tiles * ct_total;
  const int q = total >> 3, rem = total & 7;
  const int bid = (int)blockIdx.x;
  const int x = bid & 7, j = bid >> 3;
  const int t = x * q + min(x, rem) + j;
  const int per_group = kGroupRows * ct_total;
  const int grp = t / per_group;
  const int first = grp * kGroupRows;
  const int gs = min(kGroupRows, a.row_tiles - first);
  const int within = t - grp * per_group;
  const int rt = first + within % gs;
  int ct = within / gs;
  Tile T;
  T.bi = 0;
  if (a.nout > 1 && ct >= a.o[0].col_tiles) {
    T.bi = 1;
    ct -= a.o[0].col_tiles;
  }
  T.mb = (int64_t)rt * kBM;
  T.nb = (int64_t)ct * kBN;
  return T;
}

// ------------------------------------------------------------- Q tile ---
// Thread (dr = tid / 16, j = tid % 16): k-group g = dr / 2 (rows kb + 8g ..
// + 7), column half hc = dr % 2 (columns nb + 120 hc + 8j .. + 7; lane 15 of
// the DPP row only lends its chunk to lane 14).
struct QRaw {
  u32x4_t c[8];
};

__device__ __forceinline__ void q_load(QRaw& t, rsrc_t rQ, int64_t ldq, int64_t kb, int64_t col, int g, int j) {
#pragma unroll
  for (int q = 0; q < 8; ++q) t.c[q] = load_row_raw(rQ, kb + 8 * g + q, ldq, col, j);
}

// Realign (row q of the group is misaligned by (q * LD8) mod 8: the group's
// first row index is a multiple of 8 and the column a multiple of 8),
// transpose and write the 8 column segments of lane j.
template <int LD8>
__device__ __forceinline__ void q_store(const QRaw& t, char* stageQ, int64_t ldq, int64_t col, int g, int j,
                                        int J) {
  u32x4_t seg[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) seg[q] = realign_segment(t.c[q], (q * LD8) & 7, col + 8 * j, ldq, true);
  u32x4_t op[8];
  transpose8x8(seg, op);
  if (j < 15) {
    char* base = stageQ + (J >> 1) * kBlk + 256 * g + 16 * (J & 1);
#pragma unroll
    for (int e = 0; e < 8; ++e) lds_write16(base + 32 * e, op[e]);
  }
}

// ------------------------------------------------------------- P tile ---
// Unit u = 8w + i (i = 0..7) of wave w covers block u / 2, chunks 4 (u % 2)
// .. + 3; lane l fills slot l of the unit: chunk 4 (u % 2) + l / 16 of line
// sigma_inv(l % 16).
__device__ __forceinline__ void p_unit(int u, int l, int& line, int& chunk) {
  line = 16 * (u >> 1) + sigma_inv(l & 15);
  chunk = 4 * (u & 1) + (l >> 4);
}

// Aligned P: direct-to-LDS loads; chunks at or past kd read as zero.
__device__ __forceinline__ void p_load_direct(rsrc_t rP, int64_t ldp, int64_t kd, int64_t mb, int64_t kb,
                                              char* stageP, int w, int l) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int u = 8 * w + i;
    int line, chunk;
    p_unit(u, l, line, chunk);
    const int64_t k0 = kb + 8 * chunk;
    const uint32_t off = k0 < kd ? (uint32_t)(((mb + line) * ldp + k0) * 2) : kOutOfRange;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(stageP + (u >> 1) * kBlk + 1024 * (u & 1)), 16,
                                             (int)off, 0, 0, 0);
  }
}

// Misaligned P (ldp mod 8 != 0): 2-byte loads into registers.
struct PRaw {
  u32x4_t c[8];
};
__device__ __forceinline__ void p_load_regs(PRaw& t, rsrc_t rP, int64_t ldp, int64_t kd, int64_t mb, int64_t kb,
                                            int w, int l) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    int line, chunk;
    p_unit(8 * w + i, l, line, chunk);
    t.c[i] = load_kvec(rP, mb + line, ldp, kb + 8 * chunk, kd, false);
  }
}
__device__ __forceinline__ void p_store_regs(const PRaw& t, char* stageP, int w, int l) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int u = 8 * w + i;
    lds_write16(stageP + (u >> 1) * kBlk + 1024 * (u & 1) + 16 * l, t.c[i]);
  }
}

// -------------------------------------------------------------- compute ---
// One 64-deep k-step from a stage: 2 MFMA k-steps of 4 x 15 tiles.
__device__ __forceinline__ void compute_stage(const char* stage, int lane_off, int w, f32x4_t (&acc)[4][15]) {
  const char* pq = stage + lane_off;
  const char* pp = stage + kStageQ + 4 * w * kBlk + lane_off;
#pragma unroll
  for (int kk = 0; kk < 2; ++kk) {
    u32x4_t a[4], b[15];
#pragma unroll
    for (int i = 0; i < 4; ++i) a[i] = lds_read16(pp + i * kBlk + 1024 * kk);
#pragma unroll
    for (int cb = 0; cb < 15; ++cb) b[cb] = lds_read16(pq + cb * kBlk + 1024 * kk);
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int cb = 0; cb < 15; ++cb) acc[i][cb] = mfma_16x16x32(a[i], b[cb], acc[i][cb]);
  }
}

template <int LD8, bool PAL>
__device__ __forceinline__ void gemm_tile(const PreArgs& a, const Tile& T, char* smem) {
  const PreOut& O = a.o[T.bi];
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63;
  const int dr = tid >> 4, j = tid & 15;
  const int g = dr >> 1, hc = dr & 1;
  const int J = 15 * hc + j;
  const int64_t qcol = T.nb + 120 * hc;

  const rsrc_t rQ = make_rsrc(O.Q, O.qrows * O.ldq * 2);
  const rsrc_t rP = make_rsrc(O.P, a.rows * O.ldp * 2);
  const int lane_off = 256 * (l >> 4) + 16 * sigma(l & 15);

  f32x4_t acc[4][15];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int cb = 0; cb < 15; ++cb) acc[i][cb] = zero4();

  const int nks = (int)((O.kd + kBK - 1) / kBK);
  QRaw qr;
  PRaw pr;

  // prologue: stage 0
  if (PAL)
    p_load_direct(rP, O.ldp, O.kd, T.mb, 0, smem + kStageQ, w, l);
  else
    p_load_regs(pr, rP, O.ldp, O.kd, T.mb, 0, w, l);
  q_load(qr, rQ, O.ldq, 0, qcol, g, j);
  wait_vmem_all();
  q_store<LD8>(qr, smem, O.ldq, qcol, g, j, J);
  if (!PAL) p_store_regs(pr, smem + kStageQ, w, l);
  barrier_lds();

  for (int ks = 0; ks < nks; ++ks) {
    char* cur = smem + (ks & 1) * kStage;
    char* nxt = smem + ((ks + 1) & 1) * kStage;
    const bool more = ks + 1 < nks;  // uniform
    const int64_t kb = (int64_t)(ks + 1) * kBK;
    if (more) {
      if (PAL)
        p_load_direct(rP, O.ldp, O.kd, T.mb, kb, nxt + kStageQ, w, l);
      else
        p_load_regs(pr, rP, O.ldp, O.kd, T.mb, kb, w, l);
      q_load(qr, rQ, O.ldq, kb, qcol, g, j);
    }
    compute_stage(cur, lane_off, w, acc);
    if (more) {
      wait_vmem_all();
      q_store<LD8>(qr, nxt, O.ldq, qcol, g, j, J);
      if (!PAL) p_store_regs(pr, nxt + kStageQ, w, l);
      barrier_lds();
    }
  }

  // ------------------------------------------------------------ epilogue --
  // Stage the wave's 64 x 240 bf16 block in LDS with every row shifted by
  // its misalignment d = (row * ldc + nb) mod 8, so that LDS chunk k of a
  // row is global 16-byte chunk k of that row's segment.  Lane (L, G) of
  // tile (i, cb) holds rows 16i + 4G + t, column 16cb + L.
  barrier_lds();  // every wave is done with the stage buffers
  const int L = l & 15, G = l >> 4;
  const int64_t ldc = O.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = 64 * w + 16 * i + 4 * G + t;
      const int d = (int)(((T.mb + m) * ldc + T.nb) & 7);
      uint16_t* row = reinterpret_cast<uint16_t*>(smem + m * kEpiRS) + d + L;
#pragma unroll
      for (int cb = 0; cb < 15; ++cb) row[16 * cb] = (uint16_t)f32_to_bf16_rne(acc[i][cb][t]);
    }
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // this wave's LDS writes are done (rows are wave-private)
  __atomic_signal_fence(__ATOMIC_SEQ_CST);

  const rsrc_t rC = make_rsrc(O.C, a.rows * ldc * 2);
  const int64_t ncols = min64((int64_t)kBN, O.out_cols - T.nb);
  const int k = l & 31;
  for (int it = 0; it < 32; ++it) {
    const int m = 64 * w + 2 * it + (l >> 5);
    const int64_t R = T.mb + m;
    if (R >= a.rows || k > 30) continue;
    const int d = (int)((R * ldc + T.nb) & 7);
    const int n0 = 8 * k - d;  // tile column of the chunk's first element
    if (n0 >= ncols) continue;
    const u32x4_t v = lds_read16(smem + m * kEpiRS + 16 * k);
    const int64_t e0 = R * ldc + T.nb + n0;  // multiple of 8
    if (n0 >= 0 && n0 + 8 <= ncols) {
      __builtin_amdgcn_raw_buffer_store_b128(v, rC, (int)(e0 * 2), 0, 0);
    } else {
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        const int n = n0 + e;
        if (n >= 0 && n < ncols)
          __builtin_amdgcn_raw_buffer_store_b16((uint16_t)(v[e >> 1] >> (16 * (e & 1))), rC, (int)((e0 + e) * 2), 0,
                                                0);
      }
    }
  }
}

template <bool PAL>
__global__ __launch_bounds__(kPreThreads, 1) void lr_prefill_gemm_kernel(const PreArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  const Tile T = map_tile(a);
  const int64_t ld8 = a.o[T.bi].ldq & 7;
  switch (ld8) {
    case 0: gemm_tile<0, PAL>(a, T, smem); break;
    case 1: gemm_tile<1, PAL>(a, T, smem); break;
    case 2: gemm_tile<2, PAL>(a, T, smem); break;
    case 3: gemm_tile<3, PAL>(a, T, smem); break;
    case 4: gemm_tile<4, PAL>(a, T, smem); break;
    case 5: gemm_tile<5, PAL>(a, T, smem); break;
    case 6: gemm_tile<6, PAL>(a, T, smem); break;
    default: gemm_tile<7, PAL>(a, T, smem); break;
  }
}

template <bool PAL>
hipError_t launch_one(const PreArgs& args, int grid, hipStream_t stream) {
  static bool attr_set = false;
  if (!attr_set) {
    hipError_t e = hipFuncSetAttribute((const void*)lr_prefill_gemm_kernel<PAL>,
                                       hipFuncAttributeMaxDynamicSharedMemorySize, kPreLdsBytes);
    if (e != hipSuccess) return e;
    attr_set = true;
  }
  hipLaunchKernelGGL(lr_prefill_gemm_kernel<PAL>, dim3(grid), dim3(kPreThreads), kPreLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_gemm(const PreArgs& args, hipStream_t stream) {
  const int ct = args.o[0].col_tiles + (args.nout > 1 ? args.o[1].col_tiles : 0);
  const int grid = ct * args.row_tiles;
  if (grid <= 0) return hipSuccess;
  bool pal = true;
  for (int i = 0; i < args.nout; ++i) pal = pal && (args.o[i].ldp & 7) == 0;
  return pal ? launch_one<true>(args, grid, stream) : launch_one<false>(args, grid, stream);
}

bool prefill_available() {
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return false;
  return lds >= kPreLdsBytes;
}

}  // namespace lrk
