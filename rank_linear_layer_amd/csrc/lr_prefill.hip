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
// their public shapes.  Any r mod 8 and N mod 8 runs through the same code
// (the page on dimensional misalignment, "Why Smaller Is Slower? ...",
// section 3.3, traces part of the slowdown of odd ranks to misaligned
// rows; here a misaligned row costs nothing extra on the compute path).
//
// Workgroup: 8 waves (two per SIMD), tile 256 rows x 32*NB columns, 32-deep
// k-steps.  Wave (wm, wn) = (w % 4, w / 4) owns rows [64 wm, +64) and NB
// MFMA column blocks of 16: 4 x NB tiles of v_mfma_f32_16x16x32_bf16.  The
// two waves of a SIMD interleave: while one waits on LDS or a barrier the
// other keeps the matrix core busy.
//
// Every global read is a direct-to-LDS buffer load (no registers), issued
// three k-steps ahead into a ring of three raw slots:
//   P slot  256 rows x 32 k, already in MFMA operand order
//           (16-row block b, chunk c, row L at b*1024 + c*256 + L*16: one
//           operand read is 256 contiguous bytes per 16 lanes)
//   Q slot  32 rows x 33 raw 16-byte chunks of A or B, each row starting at
//           the aligned chunk that holds the tile's first column
// The MFMA B operand wants 8 consecutive k of one output column per lane,
// while A and B store the output index contiguously.  One k-step ahead of
// the MFMAs the waves gather the Q slot into Qt (same layout as the P slot,
// 16 output columns per block) with 2-byte LDS reads: element (k, n) sits at
// byte 2 (d_k + n) of raw row k, d_k = the row's misalignment, so an odd
// leading dimension needs no shifting in registers at all.
//
// An aligned P (X with K mod 8 = 0, and always T) is loaded straight into its
// slot; a misaligned X goes through registers one step ahead (2-byte loads).
//
// Grid: tiles are dealt so that each XCD (workgroup id mod 8) gets one
// contiguous run of the tile order, and the order walks groups of four row
// tiles column by column: the workgroups resident on one XCD share their P
// and Q panels in that XCD's L2.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

namespace {

constexpr int kThreads = kPreThreads;  // 512
constexpr int kBM = kPreBM;            // 256
constexpr int kBK = kPreKT;            // 32
constexpr int kSlotP = 16 * 1024;      // P slot: 16 blocks of 16 rows x 4 chunks
constexpr int kSlotQ = 15 * 1024;      // Q slot: 32 raw rows of up to 29 chunks (nb <= 7)
constexpr int kSlot = kSlotP + kSlotQ;
constexpr int kSlots = 4;              // ring depth: loads run three k-steps ahead
constexpr int kQt = 16 * 1024;         // gathered Q: 16 column blocks (the gather covers 256 columns)
constexpr int kQtBase = kSlots * kSlot;
constexpr int kGroupRows = 4;          // row tiles per group in the tile order
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;
static_assert(kQtBase + 2 * kQt <= kPreLdsBytes, "LDS layout");

// Geometry that depends on the tile width 32 * NB.
template <int NB>
struct Geo {
  static constexpr int kQChunks = 4 * NB + 1;  // raw chunks per Q row: 32 NB columns + one for misalignment
  static constexpr int kQRowBytes = kQChunks * 16;
  static constexpr int kQInst = (32 * kQChunks + 63) / 64;  // direct loads per Q slot
  static constexpr int kEpiPitch = kQRowBytes;               // epilogue staging row pitch
  static_assert(kQInst * 1024 <= kSlotQ, "Q slot");
  static_assert(kQInst <= 16, "two direct loads per wave cover the Q slot");
  // the gather reads columns up to 255 (+ 7 of misalignment) of the last raw row
  static_assert(31 * kQRowBytes + 2 * (255 + 7) + 2 <= kSlotQ, "gather stays inside the Q slot");
  static_assert(kBM * kEpiPitch <= kPreLdsBytes, "epilogue staging");
};

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ u32x4_t lds_read16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }
__device__ __forceinline__ uint32_t lds_read_u16(const char* p) { return *reinterpret_cast<const uint16_t*>(p); }
__device__ __forceinline__ void dma16(rsrc_t r, char* lds_wave_base, uint32_t off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, (int)off, 0, 0, 0);
}

// Column tiles of all the outputs of a launch (outputs follow one another
// in the tile order).
__host__ __device__ __forceinline__ int total_col_tiles(const PreArgs& a) {
  int n = 0;
#pragma unroll
  for (int i = 0; i < kPreMaxOut; ++i)
    if (i < a.nout) n += a.o[i].col_tiles;
  return n;
}

struct Tile {
  int bi;      // output block (0 or 1)
  int64_t mb;  // first row
  int64_t nb;  // first column
};

// Workgroup id -> tile.  XCD x (= id mod 8) receives the contiguous run
// [x*q + min(x, rem), ...) of the tile order; the order is row-tile groups of
// kGroupRows, walked column tile by column tile across both outputs.
__device__ __forceinline__ Tile map_tile(const PreArgs& a, int bn, int bid) {
  const int ct_total = total_col_tiles(a);
  const int total = a.row_tiles * ct_total;
  const int q = total >> 3, rem = total & 7;
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
#pragma unroll
  for (int i = 0; i + 1 < kPreMaxOut; ++i)
    if (i + 1 < a.nout && T.bi == i && ct >= a.o[i].col_tiles) {
      ct -= a.o[i].col_tiles;
      T.bi = i + 1;
    }
  T.mb = (int64_t)rt * kBM;
  T.nb = (int64_t)ct * bn;
  return T;
}

struct Ctx {
  rsrc_t rP, rQ;
  int64_t ldp, kd, ldq, qrows, mb, nb;
  int qcols;  // columns of Q inside this tile (<= BN; past them the rows hold other data)
  int w, l;
};

// -------------------------------------------------------------- loads ---
// Every direct load's byte offset is computed once per workgroup and then
// advanced by a uniform stride per k-step: P moves 32 columns (64 bytes) and
// Q moves 32 rows (64 * ldq bytes) per step, which keeps each row's
// misalignment, so the chunk selection of a lane never changes.

// P slot, aligned P: wave w loads 16-row blocks w and w + 8.  Lane l of a
// block fills chunk l / 16 of row l % 16; chunks at or past kd read zero.
struct PDma {
  uint32_t off0[2];  // byte offset at k-step 0 of this split
  int kcol;          // lane's first column at k-step 0
};
__device__ __forceinline__ void p_dma_init(const Ctx& c, int64_t k0, PDma& d) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t row = c.mb + 16 * (c.w + 8 * h) + (c.l & 15);
    d.off0[h] = (uint32_t)((row * c.ldp + k0 + 8 * (c.l >> 4)) * 2);
  }
  d.kcol = (int)(k0 + 8 * (c.l >> 4));
}
__device__ __forceinline__ void p_dma(const Ctx& c, const PDma& d, char* slotP, int t) {
  const bool ok = (int64_t)d.kcol + 32 * t < c.kd;
#pragma unroll
  for (int h = 0; h < 2; ++h) dma16(c.rP, slotP + (c.w + 8 * h) * 1024, ok ? d.off0[h] + 64u * t : kOutOfRange);
}

// P slot, misaligned P: the same two chunks per lane through registers.
struct PRegs {
  u32x4_t v[2];
};
__device__ __forceinline__ void p_regs_load(const Ctx& c, PRegs& p, int64_t kb) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int b = c.w + 8 * h;
    p.v[h] = load_kvec(c.rP, c.mb + 16 * b + (c.l & 15), c.ldp, kb + 8 * (c.l >> 4), c.kd, false);
  }
}
__device__ __forceinline__ void p_regs_store(const Ctx& c, const PRegs& p, char* slotP) {
#pragma unroll
  for (int h = 0; h < 2; ++h) lds_write16(slotP + (c.w + 8 * h) * 1024 + c.l * 16, p.v[h]);
}

// Q slot: 32 raw rows x (4 NB + 1) chunks in Geo::kQInst loads of 64
// chunks; wave w issues loads w and w + 8 (when they exist).  Only the
// chunks that hold the tile's qcols columns of a row are fetched.
struct QDma {
  uint32_t off0[2];  // byte offset at k-step 0 of this split
  int krow[2];       // lane's raw row at k-step 0 (k index)
  bool ok[2];        // lane fills a real chunk of a real row of the slot
};
template <int NB>
__device__ __forceinline__ void q_dma_init(const Ctx& c, int64_t k0, QDma& d) {
  constexpr int QC = Geo<NB>::kQChunks;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int i = c.w + 8 * h;
    const int s = 64 * i + c.l;
    const int row = s / QC, ch = s - row * QC;
    const int64_t e0 = (k0 + row) * c.ldq + c.nb;
    const int need = (int)(((e0 & 7) + c.qcols + 7) >> 3);
    d.ok[h] = i < Geo<NB>::kQInst && row < kBK && ch < need;
    d.off0[h] = d.ok[h] ? (uint32_t)(((e0 >> 3) + ch) * 16) : 0u;
    d.krow[h] = (int)(k0 + row);
  }
}
template <int NB>
__device__ __forceinline__ void q_dma(const Ctx& c, const QDma& d, char* slotQ, int t) {
  const uint32_t stride = (uint32_t)(64 * c.ldq);  // 32 rows of bf16
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    if (c.w + 8 * h < Geo<NB>::kQInst) {  // uniform
      const bool ok = d.ok[h] && (int64_t)d.krow[h] + 32 * t < c.qrows;
      dma16(c.rQ, slotQ + (c.w + 8 * h) * 1024, ok ? d.off0[h] + stride * (uint32_t)t : kOutOfRange);
    }
  }
}
// Direct loads one stage costs wave w (P: 2, Q: its share of kQInst).
template <int NB, bool PAL>
__device__ __forceinline__ int dma_per_stage(int w) {
  return (PAL ? 2 : 0) + (w < Geo<NB>::kQInst ? (Geo<NB>::kQInst - 1 - w) / 8 + 1 : 0);
}
// s_waitcnt vmcnt(n), n in [0, 4] (gfx9 encoding: expcnt and lgkmcnt left at max).
__device__ __forceinline__ void wait_vmem_upto(int n) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  switch (n) {
    case 0: __builtin_amdgcn_s_waitcnt(0x0F70); break;
    case 1: __builtin_amdgcn_s_waitcnt(0x0F71); break;
    case 2: __builtin_amdgcn_s_waitcnt(0x0F72); break;
    case 3: __builtin_amdgcn_s_waitcnt(0x0F73); break;
    default: __builtin_amdgcn_s_waitcnt(0x0F74); break;
  }
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// --------------------------------------------------------------- gather ---
// Qt block cb, chunk g, lane L holds the 8 k of k-group g for output column
// 16 cb + L.  Item = (g, n) for all 256 columns of the slot (columns past
// the tile width land in Qt blocks that no MFMA reads), two per thread, so
// the gather is straight-line code that the compiler can interleave with the
// MFMAs of the current step.  Consecutive lanes take consecutive columns:
// each 2-byte read instruction touches one contiguous run of a raw row.
// Columns at or past qcols are written as zero.
template <int NB>
__device__ __forceinline__ void gather(const Ctx& c, const char* slotQ, char* qt) {
  constexpr int kQRowBytes = Geo<NB>::kQRowBytes;
  // misalignment of raw row 8g + q: ((kb + 8g + q) * ldq + nb) mod 8 = (q * ldq) mod 8
  // (kb and nb are multiples of 8)
  int dq[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) dq[q] = (int)((q * c.ldq) & 7);
  const int tid = 64 * c.w + c.l;
#pragma unroll
  for (int it = 0; it < 2; ++it) {
    const int item = tid + kThreads * it;
    const int g = item >> 8, n = item & 255;
    const char* rows = slotQ + (8 * g) * kQRowBytes + 2 * n;
    uint32_t e[8];
#pragma unroll
    for (int q = 0; q < 8; ++q) e[q] = lds_read_u16(rows + q * kQRowBytes + 2 * dq[q]);
    u32x4_t v;
    v[0] = e[0] | (e[1] << 16);
    v[1] = e[2] | (e[3] << 16);
    v[2] = e[4] | (e[5] << 16);
    v[3] = e[6] | (e[7] << 16);
    if (n >= c.qcols) v = zerou4();
    lds_write16(qt + (n >> 4) * 1024 + g * 256 + (n & 15) * 16, v);
  }
}

// -------------------------------------------------------------- compute ---
template <int NB>
__device__ __forceinline__ void compute(const char* slotP, const char* qt, int wm, int wn, int lane_off,
                                        f32x4_t (&acc)[4][NB]) {
  u32x4_t a[4], b[NB];
#pragma unroll
  for (int i = 0; i < 4; ++i) a[i] = lds_read16(slotP + (4 * wm + i) * 1024 + lane_off);
#pragma unroll
  for (int j = 0; j < NB; ++j) b[j] = lds_read16(qt + (NB * wn + j) * 1024 + lane_off);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = mfma_16x16x32(a[i], b[j], acc[i][j]);
}

template <int NB, bool PAL>
__device__ __forceinline__ void gemm_tile(const PreArgs& a, const Tile& T, int ks, char* smem) {
  constexpr int BN = 32 * NB;
  const PreOut& O = a.o[T.bi];
  Ctx c;
  c.rP = make_rsrc(O.P, a.rows * O.ldp * 2);
  c.rQ = make_rsrc(O.Q, O.qrows * O.ldq * 2);
  c.ldp = O.ldp;
  c.kd = O.kd;
  c.ldq = O.ldq;
  c.qrows = O.qrows;
  c.mb = T.mb;
  c.nb = T.nb;
  c.qcols = (int)min64((int64_t)BN, O.ldq - T.nb);
  c.w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);  // wave-uniform: scalar branches
  c.l = threadIdx.x & 63;
  const int wm = c.w & 3, wn = c.w >> 2;
  const int lane_off = (c.l >> 4) * 256 + (c.l & 15) * 16;

  f32x4_t acc[4][NB];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = zero4();

  // this workgroup's k-steps: [s0, s0 + nks) of the ceil(kd / 32) steps
  const int nks_all = (int)((O.kd + kBK - 1) / kBK);
  const int s0 = ks * a.split_steps;
  const int nks = max(0, min(nks_all - s0, a.split_steps));
  const int64_t k0 = (int64_t)s0 * kBK;
  auto slot = [&](int s) { return smem + (s & (kSlots - 1)) * kSlot; };
  auto qtb = [&](int s) { return smem + kQtBase + (s & 1) * kQt; };
  PDma pd;
  QDma qd;
  if (PAL) p_dma_init(c, k0, pd);
  q_dma_init<NB>(c, k0, qd);
  auto stage_dma = [&](int s) {
    if (PAL) p_dma(c, pd, slot(s), s);
    q_dma<NB>(c, qd, slot(s) + kSlotP, s);
  };
  const int dma_w = dma_per_stage<NB, PAL>(c.w);

  // prologue: stages 0 and 1 landed, stage 0 gathered, stages 2 and 3 in flight
  PRegs pr;
  if (nks > 0) {
    if (!PAL) p_regs_load(c, pr, k0);
    stage_dma(0);
  }
  if (nks > 1) stage_dma(1);
  wait_vmem_all();
  if (!PAL && nks > 0) p_regs_store(c, pr, slot(0));
  barrier_lds();
  if (nks > 0) gather<NB>(c, slot(0) + kSlotP, qtb(0));
  if (!PAL && nks > 1) p_regs_load(c, pr, k0 + kBK);
  if (nks > 2) stage_dma(2);
  if (nks > 3) stage_dma(3);
  if (!PAL && nks > 1) {
    wait_vmem_all();
    p_regs_store(c, pr, slot(1));
  }
  barrier_lds();

  for (int s = 0; s < nks; ++s) {
    // misaligned P: stage s + 2 travels through registers during this step
    if (!PAL && s + 2 < nks) p_regs_load(c, pr, k0 + (int64_t)(s + 2) * kBK);
    compute<NB>(slot(s), qtb(s), wm, wn, lane_off, acc);
    // next stage's operand (past the last stage this reads a consumed slot
    // and fills a Qt buffer nothing reads again)
    gather<NB>(c, slot(s + 1) + kSlotP, qtb(s + 1));
    // stage s + 2 has landed; stage s + 3 (issued one step later) may still
    // be in flight.  The misaligned P path drains everything.
    if (PAL && s + 3 < nks)
      wait_vmem_upto(dma_w);
    else
      wait_vmem_all();
    if (!PAL && s + 2 < nks) p_regs_store(c, pr, slot(s + 2));
    barrier_lds();
    // slot s is free: every wave is past compute(s) and gathered s earlier
    if (s + 4 < nks) stage_dma(s + 4);
  }

  // ------------------------------------------------------------ epilogue --
  if (a.splits > 1) {
    // fp32 partial of this k-split: [ks][rows][ldpart], summed in split order
    // and rounded by lr_prefill_reduce_kernel.  Lane (L, G) of tile (i, j)
    // holds rows 64 wm + 16 i + 4 G + t, column 16 (NB wn + j) + L.
    const int L = c.l & 15, G = c.l >> 4;
    float* part = O.part + (int64_t)ks * a.rows * O.ldpart;
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        const int64_t m = T.mb + 64 * wm + 16 * i + 4 * G + t;
#pragma unroll
        for (int j = 0; j < NB; ++j) {
          const int64_t n = T.nb + 16 * (NB * wn + j) + L;
          if (m < a.rows && n < O.out_cols) part[m * O.ldpart + n] = acc[i][j][t];
        }
      }
    return;
  }
  // Stage the 256 x BN bf16 tile in LDS with every row shifted by its
  // misalignment d = (row * ldc + nb) mod 8, so that LDS chunk k of a row is
  // global 16-byte chunk k of that row's segment.  Lane (L, G) of tile
  // (i, j) holds rows 64 wm + 16 i + 4 G + t, column 16 (NB wn + j) + L.
  const int L = c.l & 15, G = c.l >> 4;
  const int64_t ldc = O.ldc;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int m = 64 * wm + 16 * i + 4 * G + t;
      const int d = (int)(((T.mb + m) * ldc + T.nb) & 7);
      uint16_t* row = reinterpret_cast<uint16_t*>(smem + m * Geo<NB>::kEpiPitch) + d + 16 * NB * wn + L;
#pragma unroll
      for (int j = 0; j < NB; ++j) row[16 * j] = (uint16_t)f32_to_bf16_rne(acc[i][j][t]);
    }
  }
  barrier_lds();

  const rsrc_t rC = make_rsrc(O.C, a.rows * ldc * 2);
  const int ncols = (int)min64((int64_t)BN, O.out_cols - T.nb);
  constexpr int kQChunks = Geo<NB>::kQChunks;
  constexpr int nitems = kBM * kQChunks;
  for (int item = threadIdx.x; item < nitems; item += kThreads) {
    const int m = item / kQChunks, k = item - m * kQChunks;
    const int64_t R = T.mb + m;
    if (R >= a.rows) continue;
    const int d = (int)((R * ldc + T.nb) & 7);
    const int n0 = 8 * k - d;  // tile column of the chunk's first element
    if (n0 >= ncols) continue;
    const u32x4_t v = lds_read16(smem + m * Geo<NB>::kEpiPitch + 16 * k);
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

template <int NB, bool PAL>
__global__ __launch_bounds__(kThreads, 1) void lr_prefill_gemm_kernel(const PreArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  // workgroup -> (tile, k-split): consecutive ids are different tiles of one
  // split, so the XCD dealing of tiles is the same for every split
  const int tiles = a.row_tiles * total_col_tiles(a);
  const int ks = (int)blockIdx.x / tiles;
  const Tile T = map_tile(a, 32 * NB, (int)blockIdx.x - ks * tiles);
  gemm_tile<NB, PAL>(a, T, ks, smem);
}

// Y (or T) = bf16(sum over k-splits of the fp32 partials, in split order).
// Thread -> 4 consecutive columns of one row.
__global__ __launch_bounds__(256) void lr_prefill_reduce_kernel(const float* part, int splits, int64_t rows,
                                                               int64_t cols, int64_t ldpart, uint16_t* C,
                                                               int64_t ldc) {
  const int64_t q = (cols + 3) / 4;
  const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
  if (idx >= rows * q) return;
  const int64_t m = idx / q, n = (idx - m * q) * 4;
  const float* p = part + m * ldpart + n;
  f32x4_t sum = *reinterpret_cast<const f32x4_t*>(p);
  for (int s = 1; s < splits; ++s) sum += *reinterpret_cast<const f32x4_t*>(p + (int64_t)s * rows * ldpart);
  uint16_t* c = C + m * ldc + n;
  if (n + 4 <= cols && ((m * ldc + n) & 3) == 0) {
    uint2 v;
    v.x = pack_bf16x2(sum[0], sum[1]);
    v.y = pack_bf16x2(sum[2], sum[3]);
    *reinterpret_cast<uint2*>(c) = v;
  } else {
#pragma unroll
    for (int e = 0; e < 4; ++e)
      if (n + e < cols) c[e] = (uint16_t)f32_to_bf16_rne(sum[e]);
  }
}

template <int NB, bool PAL>
hipError_t launch_one(const PreArgs& args, int grid, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  {
    const hipError_t e = ensure_dynamic_lds((const void*)lr_prefill_gemm_kernel<NB, PAL>, kPreLdsBytes, attr_done);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((lr_prefill_gemm_kernel<NB, PAL>), dim3(grid), dim3(kThreads), kPreLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_gemm(const PreArgs& args, hipStream_t stream) {
  const int ct = total_col_tiles(args);
  const int grid = ct * args.row_tiles * args.splits;
  if (grid <= 0) return hipSuccess;
  bool pal = true;
  for (int i = 0; i < args.nout; ++i) pal = pal && (args.o[i].ldp & 7) == 0;
  switch (args.nb) {
    case 6: return pal ? launch_one<6, true>(args, grid, stream) : launch_one<6, false>(args, grid, stream);
    case 7: return pal ? launch_one<7, true>(args, grid, stream) : launch_one<7, false>(args, grid, stream);
    default: return hipErrorInvalidValue;
  }
}

hipError_t launch_prefill_reduce(const float* part, int splits, int64_t rows, int64_t cols, int64_t ldpart,
                                 uint16_t* C, int64_t ldc, hipStream_t stream) {
  const int64_t items = rows * ((cols + 3) / 4);
  if (items <= 0) return hipSuccess;
  hipLaunchKernelGGL(lr_prefill_reduce_kernel, dim3((unsigned)((items + 255) / 256)), dim3(256), 0, stream, part,
                     splits, rows, cols, ldpart, C, ldc);
  return hipGetLastError();
}

bool prefill_available() {
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return false;
  return lds >= kPreLdsBytes;
}

}  // namespace lrk
