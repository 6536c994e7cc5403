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
// their public shapes.  Any r mod 8, N mod 8 and K mod 8 runs through the
// same instructions (the page on dimensional misalignment, "Why Smaller Is
// Slower? ...", section 3.3, traces part of the slowdown of odd ranks to
// misaligned rows): every row is loaded from its exact first element.
//
// Workgroup: 8 waves (two per SIMD), tile 256 rows x 32*NB columns, 32-deep
// k-steps.  Wave (wm, wn) = (w % 4, w / 4) owns rows [64 wm, +64) and NB
// MFMA column blocks of 16: 4 x NB tiles of v_mfma_f32_16x16x32_bf16.  The
// two waves of a SIMD alternate between barriers: one issues its MFMAs
// while the other reads its next operands from LDS.
//
// Every global read is a direct-to-LDS 16-byte buffer load (no registers)
// that starts at the exact element it needs: gfx950's buffer loads return
// the 16 bytes at any 2-byte aligned offset.  Loads run four k-steps ahead
// into a ring of five slots, each holding
//   P  256 rows x 32 k of X or T in 16-row blocks of 1 KB; chunk c of row
//      L at 16 (4 L + (c ^ (L / 4 mod 4))): a lane quad loads one row's 64
//      bytes, and the MFMA operand reads are free of bank conflicts
//   Q  32 rows x 32*NB columns of A or B, row-major with a pitch of
//      64 NB + 32 bytes, k-row 8 kq + 4 h + q stored at slot row
//      16 h + 4 kq + q.
// The MFMA B operand wants 8 consecutive k of one output column per lane,
// while A and B store the output index contiguously: the transposing LDS
// read (ds_read_b64_tr_b16) delivers it from Q directly.  Its 16-lane
// groups read 4 slot rows each; with the row order above a half-wave reads
// 8 consecutive slot rows, whose pitch (an odd multiple of 32 bytes) puts
// them in 8 different 32-byte bank groups.
//
// The buffer range check zeroes a dword that reaches past the range end, so
// an unaligned load loses a matrix's last element when the matrix ends on a
// dword boundary; and a P row chunk that straddles the reduction length
// holds the next row's first elements.  The one k-step of a tile where
// either happens patches its slot after the loads land (a scalar load for
// the last element, zeros past the reduction length) behind one more
// barrier.
//
// Grid: tiles are dealt so that each XCD (workgroup id mod 8) gets one
// contiguous run of the tile order, and the order walks groups of four row
// tiles column by column: the workgroups resident on one XCD share their P
// and Q panels in that XCD's L2.
#include <type_traits>

#include "lr_device.h"
#include "lr_kernels.h"
#include "lr_ldsops.h"

namespace lrk {

namespace {

constexpr int kThreads = kPreThreads;  // 512
constexpr int kBM = kPreBM;            // 256
constexpr int kBK = kPreKT;            // 32
constexpr int kSlotP = 16 * 1024;      // P: 16 blocks of 16 rows x 4 chunks
constexpr int kSlot = kPreSlotBytes;   // P + Q of the widest tile
constexpr int kSlots = kPreSlots;      // ring depth: loads run kSlots - 1 k-steps ahead
constexpr int kAhead = kSlots - 1;
constexpr int kGroupRows = 4;          // row tiles per group in the tile order
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;
static_assert(kSlots * kSlot + 1024 <= kPreLdsBytes, "LDS layout: the ring and a spare 1 KB");
static_assert(kAhead == 4, "wait_stages covers three stages in flight");

// Geometry that depends on the tile width 32 * NB.
template <int NB>
struct Geo {
  static constexpr int kQPitch = 64 * NB + 32;              // bytes per Q slot row (an odd multiple of 32)
  static constexpr int kQInst = 2 * NB + 1;                 // 1 KB direct loads per Q slot (32 rows)
  static constexpr int kQChunks = 4 * NB;                   // 16-byte chunks of data per Q row
  static constexpr int kEpiPitch = (4 * NB + 1) * 16;       // epilogue staging row pitch
  static_assert(32 * kQPitch == 1024 * kQInst, "Q slot is a whole number of loads");
  static_assert(kSlotP + 1024 * kQInst <= kSlot, "Q slot");
  static_assert(kQInst <= 16, "two direct loads per wave cover the Q slot");

  static_assert(kBM * kEpiPitch <= kPreLdsBytes, "epilogue staging");
};


__device__ __forceinline__ u32x4_t lds_read16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }
typedef int i32x4_t __attribute__((ext_vector_type(4)));
typedef short s16x4_t __attribute__((ext_vector_type(4)));
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
}
// Raw buffer resource (base, no stride, `bytes` rounded up to whole dwords).
__device__ __forceinline__ i32x4_t rsrc4(const void* base, int64_t bytes) {
  const uint64_t b = (uint64_t)(uintptr_t)base;
  return i32x4_t{(int)(uint32_t)b, (int)((uint32_t)(b >> 32) & 0xFFFFu), (int)(uint32_t)((bytes + 3) & ~(int64_t)3),
                 kRsrcFlags};
}
// 16 bytes per lane from byte offset `off` of the buffer into LDS at
// lds_base + 16 * lane.  Issued from asm: the compiler then does not count
// it among the stores to LDS that an LDS read has to wait for (the loop
// waits for its loads with explicit counts).  No register receives data.
__device__ __forceinline__ void dma16a(const i32x4_t& r, uint32_t lds_base, uint32_t off) {
  // one wait state between the write of M0 and the load that reads it
  asm volatile("s_nop 0\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds" ::"v"(off), "s"(r), "{m0}"(lds_base) : "memory");
}
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }
// Transposing LDS read (ds_read_b64_tr_b16): within a 16-lane group, lane
// 4 q + c reads 8 bytes (row q, columns 4 c .. 4 c + 3 of a 4 x 16 bf16
// tile) and receives the 4 values of column (lane mod 16).
typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
typedef __attribute__((address_space(3))) s16x4_t lds_s16x4_t;
__device__ __forceinline__ u32x2_t lds_read_tr(const lds_s16x4_t* p) {
  return __builtin_bit_cast(u32x2_t, __builtin_amdgcn_ds_read_tr16_b64_v4i16(const_cast<lds_s16x4_t*>(p)));
}
// Slot row of k-row kr (0..31) of a Q slot.
__host__ __device__ __forceinline__ int q_slot_row(int kr) { return 16 * ((kr >> 2) & 1) + 4 * (kr >> 3) + (kr & 3); }

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

// Workgroup id -> (tile, k-split).  The units of a launch are ordered
// split by split, and within a split row-tile groups of kGroupRows walked
// column tile by column tile across all the outputs.  XCD x (= id mod 8)
// receives the contiguous run [x*q + min(x, rem), ...) of that order, so
// the workgroups resident on one XCD share P and Q panels, and with a
// k-split each XCD reads the k-range of one or two splits only.
__device__ __forceinline__ Tile map_unit(const PreArgs& a, int bn, int bid, int& ks) {
  const int ct_total = total_col_tiles(a);
  const int tiles = a.row_tiles * ct_total;
  const int total = tiles * a.splits;
  const int q = total >> 3, rem = total & 7;
  const int x = bid & 7, j = bid >> 3;
  const int u = x * q + min(x, rem) + j;
  ks = u / tiles;
  const int t = u - ks * tiles;
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
  i32x4_t rP, rQ;
  const uint16_t* P;
  const uint16_t* Q;
  int64_t rows, ldp, kd, ldq, qrows, mb, nb;
  int qcols;  // columns of Q inside this tile (<= BN; past them the rows hold other data)
  int w, l;
};

// -------------------------------------------------------------- loads ---
// Every direct load's byte offset is computed once per workgroup and then
// advanced by a uniform stride per k-step: P moves 32 columns (64 bytes) and
// Q moves 32 rows (64 * ldq bytes) per step.

// P slot: wave w loads 16-row blocks w and w + 8.  Lane l of a block fills
// chunk l / 16 of row l % 16 from its exact first element; chunks that start
// at or past kd read zero, rows past the matrix fall outside the range.
struct PDma {
  uint32_t off0[2];  // byte offset at k-step 0 of this split
  int kcol;          // lane's first column at k-step 0
};
// Position (16-byte unit) of chunk c of row L in a 16-row P block: the four
// lanes of a quad load one row's 64 bytes (whole row segments per request),
// and the XOR by L / 4 keeps the MFMA operand reads (16 lanes, one chunk of
// 16 rows) free of bank conflicts.
__device__ __forceinline__ int p_pos(int L, int c) { return 4 * L + (c ^ ((L >> 2) & 3)); }
// Row and chunk that lane l of a P load fills (the inverse of p_pos).
__device__ __forceinline__ int p_row(int l) { return l >> 2; }
__device__ __forceinline__ int p_chunk(int l) { return (l & 3) ^ ((l >> 4) & 3); }
__device__ __forceinline__ void p_dma_init(const Ctx& c, int64_t k0, PDma& d) {
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int64_t row = c.mb + 16 * (c.w + 8 * h) + p_row(c.l);
    d.off0[h] = (uint32_t)((row * c.ldp + k0 + 8 * p_chunk(c.l)) * 2);
  }
  d.kcol = (int)(k0 + 8 * p_chunk(c.l));
}
__device__ __forceinline__ void p_dma(const Ctx& c, const PDma& d, char* slotP, int t) {
  const bool ok = (int64_t)d.kcol + 32 * t < c.kd;
#pragma unroll
  for (int h = 0; h < 2; ++h) dma16a(c.rP, lds_addr(slotP + (c.w + 8 * h) * 1024), ok ? d.off0[h] + 64u * t : kOutOfRange);
}

// Q slot: Geo::kQInst loads of 1 KB; wave w issues loads w and w + 8 (when
// they exist).  Lane l of load u lands at slot byte 1024 u + 16 l, i.e. slot
// row R, chunk ch; it fetches chunk ch of k-row kr(R) from its exact first
// element.  Chunks in the row padding, past the tile's qcols columns or past
// the matrix's rows read zero.
struct QDma {
  uint32_t off0[2];  // byte offset at k-step 0 of this split
  int krow[2];       // lane's k-row at k-step 0
  bool ok[2];        // lane fills a real chunk of the slot
};
template <int NB>
__device__ __forceinline__ void q_dma_init(const Ctx& c, int64_t k0, QDma& d) {
  constexpr int kPitch = Geo<NB>::kQPitch;
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int u = c.w + 8 * h;
    const int pos = 1024 * u + 16 * c.l;
    const int R = pos / kPitch, ch = (pos - R * kPitch) >> 4;
    const int kr = 8 * ((R >> 2) & 3) + 4 * (R >> 4) + (R & 3);
    d.ok[h] = u < Geo<NB>::kQInst && ch < Geo<NB>::kQChunks && 8 * ch < c.qcols;
    d.krow[h] = (int)(k0 + kr);
    d.off0[h] = d.ok[h] ? (uint32_t)(((k0 + kr) * c.ldq + c.nb + 8 * ch) * 2) : 0u;
  }
}
// Direct loads per wave and k-step: two of P and D - 2 of Q, one for each Q
// load wave w has (loads w and w + 8 of the slot, where they exist).  The
// spare 1 KB of LDS stays as a target for loads that fill nothing.
template <int NB, int D>
__device__ __forceinline__ void q_dma(const Ctx& c, const QDma& d, char* slotQ, char* dummy, int t) {
  const uint32_t stride = (uint32_t)(64 * c.ldq);  // 32 rows of bf16
#pragma unroll
  for (int h = 0; h < D - 2; ++h) {
    const bool real = c.w + 8 * h < Geo<NB>::kQInst;  // uniform
    const bool ok = real && d.ok[h] && (int64_t)d.krow[h] + 32 * t < c.qrows;
    dma16a(c.rQ, lds_addr(real ? slotQ + (c.w + 8 * h) * 1024 : dummy), ok ? d.off0[h] + stride * (uint32_t)t : kOutOfRange);
  }
}
// Wait until at most n stages of this wave's loads (D per stage) are in
// flight (n <= 3).
template <int D>
__device__ __forceinline__ void wait_stages(int n) {
  constexpr int d = D;
  switch (n) {
    case 0: wait_vm_dyn(0); break;
    case 1: wait_vm_dyn(d); break;
    case 2: wait_vm_dyn(2 * d); break;
    default: wait_vm_dyn(3 * d); break;
  }
}

// The k-step of a tile whose slot needs patching after its loads land:
//  * Q with an odd leading dimension: the matrix's last element (row
//    qrows - 1, column ldq - 1), in the tile holding that column;
//  * P with kd mod 8 != 0: the chunks that straddle kd hold the next row's
//    first elements (cleared), and the matrix's last element (set).
template <int NB>
__device__ __forceinline__ void patch_slot(const Ctx& c, char* slotP, char* slotQ, int64_t kstep0, bool fix_q,
                                           bool fix_p) {
  if (fix_q && c.w == 0 && c.l == 0) {
    const int kr = (int)(c.qrows - 1 - kstep0);
    const int n = (int)(c.ldq - 1 - c.nb);
    *reinterpret_cast<uint16_t*>(slotQ + q_slot_row(kr) * Geo<NB>::kQPitch + 2 * n) =
        (uint16_t)scalar_elem(c.Q, c.qrows * c.ldq - 1);
  }
  if (fix_p) {
    const int64_t kk = kstep0 + 8 * p_chunk(c.l);
    if (kk < c.kd && kk + 8 > c.kd) {
      const int valid = (int)(c.kd - kk);  // 1 .. 7 elements of this chunk lie below kd
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const int64_t row = c.mb + 16 * (c.w + 8 * h) + p_row(c.l);
        char* p = slotP + (c.w + 8 * h) * 1024 + 16 * c.l;
        u32x4_t v = lds_read16(p);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
          // dword i holds elements 2 i and 2 i + 1
          const uint32_t keep = 2 * i + 1 < valid ? 0xFFFFFFFFu : (2 * i < valid ? 0x0000FFFFu : 0u);
          v[i] &= keep;
        }
        if (row == c.rows - 1 && c.ldp == c.kd) {
          const int e = valid - 1;
          const uint32_t x = scalar_elem(c.P, c.rows * c.ldp - 1) << (16 * (e & 1));
          const uint32_t m = 0xFFFFu << (16 * (e & 1));
#pragma unroll
          for (int i = 0; i < 4; ++i)
            if (i == (e >> 1)) v[i] = (v[i] & ~m) | x;
        }
        lds_write16(p, v);
      }
    }
  }
}

// -------------------------------------------------------------- compute ---
// Barrier that no instruction crosses: the MFMAs carry no memory dependence,
// so without the scheduling fences the compiler would move them past the
// barriers that separate the two wave groups' turns.
__device__ __forceinline__ void turn_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  barrier_lds();
  __builtin_amdgcn_sched_barrier(0);
}
// The barrier between a group's operand reads and its MFMAs: it does not
// wait for those reads (the MFMAs wait for the operands they use), only for
// the other group to finish its MFMAs' issue.
__device__ __forceinline__ void handoff_barrier() {
  __builtin_amdgcn_sched_barrier(0);
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_sched_barrier(0);
}

// The operands of one k-step, in registers until the MFMAs consume them.
template <int NB>
struct Ops {
  u32x4_t a[4], b[NB];
};
// The operand reads of one k-step: the compiler waits for each before the
// first MFMA that uses it.  (The direct loads are issued from asm, so the
// compiler does not make these reads wait for the loads still in flight
// into other slots.)
template <int NB>
__device__ __forceinline__ void read_p(const char* slotP, int wm, int l, Ops<NB>& o) {
  const int off = 16 * p_pos(l & 15, l >> 4);  // row l % 16, chunk l / 16
#pragma unroll
  for (int i = 0; i < 4; ++i) o.a[i] = lds_read16(slotP + (4 * wm + i) * 1024 + off);
}
template <int NB>
__device__ __forceinline__ void read_q(const char* slotQ, int wn, int l, Ops<NB>& o) {
  // lane l = 16 kq + 4 q + c reads slot rows l / 4 and 16 + l / 4, bytes
  // 8 c of each 32-byte column group
  const uint32_t a = lds_addr(slotQ) + (uint32_t)((l >> 2) * Geo<NB>::kQPitch + 8 * (l & 3) + 32 * NB * wn);
  const lds_s16x4_t* q = (const lds_s16x4_t*)(uintptr_t)a;
#pragma unroll
  for (int j = 0; j < NB; ++j) {
    // 8-byte elements: column group j at byte 32 j, the second half 16 slot rows further
    const u32x2_t lo = lds_read_tr(q + 4 * j), hi = lds_read_tr(q + 2 * Geo<NB>::kQPitch + 4 * j);
    o.b[j] = u32x4_t{lo[0], lo[1], hi[0], hi[1]};
  }
}
template <int NB>
__device__ __forceinline__ void mma(const Ops<NB>& o, f32x4_t (&acc)[4][NB]) {
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < NB; ++j) acc[i][j] = mfma_16x16x32(o.a[i], o.b[j], acc[i][j]);
}

template <int NB>
__device__ __forceinline__ void gemm_tile(const PreArgs& a, const Tile& T, int ks, char* smem) {
  constexpr int BN = 32 * NB;
  const PreOut& O = a.o[T.bi];
  Ctx c;
  c.rP = rsrc4(O.P, a.rows * O.ldp * 2);
  c.rQ = rsrc4(O.Q, O.qrows * O.ldq * 2);
  c.P = O.P;
  c.Q = O.Q;
  c.rows = a.rows;
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
  auto slot = [&](int s) { return smem + (s % kSlots) * kSlot; };
  PDma pd;
  QDma qd;
  p_dma_init(c, k0, pd);
  q_dma_init<NB>(c, k0, qd);
  // the k-steps (relative to this split) that need a patch, else -1
  const bool q_last_tile = (c.ldq & 1) && T.nb + c.qcols == c.ldq;
  const int q_fix = q_last_tile && c.qrows - 1 >= k0 ? (int)((c.qrows - 1 - k0) / kBK) : -1;
  const int p_fix = (c.kd & 7) && c.kd - 1 >= k0 ? (int)((c.kd - 1 - k0) / kBK) : -1;

  // The two waves of a SIMD take turns (waves 0-3 and 4-7, one of each per
  // SIMD): between two barriers one group issues its MFMAs while the other
  // issues its next operand reads and the next loads, so the matrix cores
  // stay busy while the LDS reads of the other group are in flight.  The
  // barrier between a group's reads and its MFMAs (the hand-off) does not
  // wait for the reads; the barrier that opens a k-step does, and every slot
  // is refilled only after one of those.  Group 0 reads stage t, then
  // multiplies it; group 1 multiplies stage t - 1 while group 0 reads t, and
  // reads t while group 0 multiplies.  Both groups meet the same barriers:
  //   wait for stage t; barrier; [patch; barrier]; X; barrier; Y
  //   group 0: X = read t + loads of t + 4, Y = MFMAs of t
  //   group 1: X = MFMAs of t - 1,          Y = read t + loads of t + 4
  // Stage t's slot was last read by group 1 before the first barrier of
  // iteration t + 1, so both groups refill it (with stage t + 5) after that.
  // The loop is instantiated for the wave's load count D (2, 3 or 4), so
  // that every wait count is a constant.
  const int grp = c.w >> 2;
  auto run = [&](auto dtag) {
    constexpr int D = decltype(dtag)::value;
    auto stage_dma = [&](int s) {
      p_dma(c, pd, slot(s), s);
      q_dma<NB, D>(c, qd, slot(s) + kSlotP, smem + kSlots * kSlot, s);
    };
    Ops<NB> ops;
    for (int t = 0; t < kAhead && t < nks; ++t) stage_dma(t);
    // wait for stage s, publish it, patch it where needed; `steady`: three
    // later stages are in flight (a constant wait, no branch on the count)
    auto arrive = [&](int s, bool steady) {
      wait_stages<D>(steady ? kAhead - 1 : min(kAhead - 1, nks - 1 - s));
      turn_barrier();
      if (s == q_fix || s == p_fix) {  // uniform
        patch_slot<NB>(c, slot(s), slot(s) + kSlotP, k0 + (int64_t)s * kBK, s == q_fix, s == p_fix);
        turn_barrier();
      }
    };
    // the P reads go out first, the next loads are issued while they are in
    // flight, and the B reads come last; nothing here waits for them
    auto fetch = [&](int s) {
      read_p<NB>(slot(s), wm, c.l, ops);
      if (s + kAhead < nks) stage_dma(s + kAhead);
      read_q<NB>(slot(s) + kSlotP, wn, c.l, ops);
    };
    const int steady_end = nks - (kAhead - 1);  // k-steps with three later stages in flight
    if (grp == 0) {
      int s = 0;
      for (; s < steady_end; ++s) {
        arrive(s, true);
        fetch(s);
        handoff_barrier();
        mma<NB>(ops, acc);
      }
      for (; s < nks; ++s) {
        arrive(s, false);
        fetch(s);
        handoff_barrier();
        mma<NB>(ops, acc);
      }
      turn_barrier();
    } else if (nks > 0) {
      arrive(0, steady_end > 0);
      handoff_barrier();
      fetch(0);
      int s = 1;
      for (; s < steady_end; ++s) {
        arrive(s, true);
        mma<NB>(ops, acc);
        handoff_barrier();
        fetch(s);
      }
      for (; s < nks; ++s) {
        arrive(s, false);
        mma<NB>(ops, acc);
        handoff_barrier();
        fetch(s);
      }
      turn_barrier();
      mma<NB>(ops, acc);
    } else {
      turn_barrier();
    }
  };
  if constexpr (Geo<NB>::kQInst > 8) {
    if (c.w + 8 < Geo<NB>::kQInst)  // uniform
      run(std::integral_constant<int, 4>{});
    else
      run(std::integral_constant<int, 3>{});
  } else {
    if (c.w < Geo<NB>::kQInst)  // uniform
      run(std::integral_constant<int, 3>{});
    else
      run(std::integral_constant<int, 2>{});
  }

  // ------------------------------------------------------------ epilogue --
  // Columns at or past qcols are 0 (a chunk that straddles qcols brought in
  // the next row's first elements).
  const int L = c.l & 15, G = c.l >> 4;
#pragma unroll
  for (int j = 0; j < NB; ++j)
    if (16 * (NB * wn + j) + L >= c.qcols)
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i][j] = zero4();
  if (a.splits > 1) {
    // fp32 partial of this k-split: [ks][rows][ldpart], summed in split order
    // and rounded by lr_prefill_reduce_kernel.  Lane (L, G) of tile (i, j)
    // holds rows 64 wm + 16 i + 4 G + t, column 16 (NB wn + j) + L.
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
  // Every wave is past its last LDS read: the ring memory is free.
  barrier_lds();
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
  constexpr int kQChunks = Geo<NB>::kQChunks + 1;
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

template <int NB>
__global__ __launch_bounds__(kThreads, 1) void lr_prefill_gemm_kernel(const PreArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int ks;
  const Tile T = map_unit(a, 32 * NB, (int)blockIdx.x, ks);
  gemm_tile<NB>(a, T, ks, smem);
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

template <int NB>
hipError_t launch_one(const PreArgs& args, int grid, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  {
    const hipError_t e = ensure_dynamic_lds((const void*)lr_prefill_gemm_kernel<NB>, kPreLdsBytes, attr_done);
    if (e != hipSuccess) return e;
  }
  hipLaunchKernelGGL((lr_prefill_gemm_kernel<NB>), dim3(grid), dim3(kThreads), kPreLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_prefill_gemm(const PreArgs& args, hipStream_t stream) {
  const int ct = total_col_tiles(args);
  const int grid = ct * args.row_tiles * args.splits;
  if (grid <= 0) return hipSuccess;
  switch (args.nb) {
    case 2: return launch_one<2>(args, grid, stream);
    case 3: return launch_one<3>(args, grid, stream);
    case 4: return launch_one<4>(args, grid, stream);
    case 6: return launch_one<6>(args, grid, stream);
    case 7: return launch_one<7>(args, grid, stream);
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
