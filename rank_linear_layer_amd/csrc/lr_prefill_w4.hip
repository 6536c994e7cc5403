// Prefill GEMM with one wave per SIMD and 128 x 128 wave tiles (M > 16,
// 16-byte aligned P).
//
// Same product, phases and tile walk as lr_prefill.hip (phase 1 T = X . A
// with the rank padded on chip, phase 2 Y = T . B; k-split partials), laid
// out for the way gfx950 moves data:
//  * L2 -> LDS loads run at full rate only when each instruction covers
//    whole 128-byte lines.  A k-stage is therefore 64 deep, so one row of P
//    is exactly one line; a direct-to-LDS load of 8 rows x 128 B fills the
//    P slot with an XOR swizzle (chunk c of row R at position
//    8 R + (c ^ ((R / 2) mod 8))) that keeps the MFMA operand reads free of
//    bank conflicts.
//  * The weight operand (A or B, output index contiguous) is read with
//    16-byte loads into registers: lanes 0-31 take 32 consecutive chunks of
//    one row, lanes 32-63 the same chunks 8 rows further.  Each load starts
//    exactly at its 8 elements, wherever the row begins: gfx950's buffer
//    loads return the 16 bytes at any 2-byte aligned offset (checked on
//    MI355X, at the same streaming bandwidth as aligned loads), so an odd
//    rank or width takes the same instructions as an aligned one and no
//    code depends on the leading dimension modulo 8.  One exception, at the
//    matrix's end: the buffer range check zeroes a dword that reaches past
//    the range, so when the matrix ends on a dword boundary the lane whose
//    load starts 2 bytes past one and covers the last element reads it as
//    zero; that element is patched from a scalar load, in the stages whose
//    rows can reach it only.  Each lane then
//    transposes its 8 rows x 8 columns block with v_perm_b32 and writes 8
//    operand vectors (8 k of one column) into the Qt slot, whose 16-column
//    groups are XOR-permuted so that both these writes and the MFMA reads
//    are conflict free.
//  * Four waves, one per SIMD, each own a 128 x 128 quarter of the 256 x 256
//    tile: 16 v_mfma_f32_32x32x16_bf16 accumulators (256 AGPRs), the largest
//    wave tile the register file holds, which minimises LDS operand traffic
//    per flop.
//
// LDS holds three P slots and two Qt slots (160 KB).  P of stage s + 3 is
// requested after the barrier of stage s (two stages to arrive), the weight
// rows of stage s + 2 at the start of stage s into one of two register sets
// (a little over one stage).  The cost per 64-deep stage measured on MI355X
// is about 3600 cycles for 64 MFMAs of 32 cycles each; the plan picks this
// kernel where its 256-wide tiles make that cheaper than the two-wave one.
#include "lr_device.h"
#include "lr_kernels.h"

// Optional per-stage timestamps (shader clock) of the first eight workgroups
// of launches with LR_PREFILL_TRACE workgroups, compiled in only with
// -DLR_PREFILL_TRACE=<grid>; lr_prefill_trace_read() copies them out.
#ifdef LR_PREFILL_TRACE
__device__ uint64_t g_w4trace[8 * 4 * 64 * 8];
extern "C" int lr_prefill_trace_read(void* host) {
  return (int)hipMemcpyFromSymbol(host, HIP_SYMBOL(g_w4trace), sizeof(g_w4trace));
}
#define W4_TRACE(k)                                                                            \
  do {                                                                                         \
    __builtin_amdgcn_sched_barrier(0);                                                         \
    if (gridDim.x == LR_PREFILL_TRACE && blockIdx.x < 8 && s < 64 && (threadIdx.x & 63) == 0)  \
      g_w4trace[((blockIdx.x * 4 + w) * 64 + s) * 8 + (k)] = __builtin_amdgcn_s_memtime();      \
    __builtin_amdgcn_sched_barrier(0);                                                         \
  } while (0)
// tile-level points (start, after the prologue, after the stages, end) go to stage slot 63
#define W4_TRACE_TILE(k)                                                                      \
  do {                                                                                        \
    __builtin_amdgcn_sched_barrier(0);                                                        \
    if (gridDim.x == LR_PREFILL_TRACE && blockIdx.x < 8 && (threadIdx.x & 63) == 0)           \
      g_w4trace[((blockIdx.x * 4 + w) * 64 + 63) * 8 + (k)] = __builtin_amdgcn_s_memtime();   \
    __builtin_amdgcn_sched_barrier(0);                                                        \
  } while (0)
#else
#define W4_TRACE(k) \
  do {              \
  } while (0)
#define W4_TRACE_TILE(k) \
  do {                   \
  } while (0)
#endif

namespace lrk {

namespace {

constexpr int kThreads = 256;
constexpr int kBM = 256;
constexpr int kBN = 256;
constexpr int kPSlot = kBM * 64 * 2;   // 32 KB: 256 rows x 64 k
constexpr int kQtSlot = kBN * 64 * 2;  // 32 KB: 256 columns x 64 k
constexpr int kStageChunks = kBN / 8 + 1;  // staged output row: 256 columns + room for misalignment
constexpr int kStageRowBytes = kStageChunks * 16;
constexpr int kGroupRows = 4;
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;

constexpr int kPSlots = 3;
constexpr int kQtBase = kPSlots * kPSlot;
// three P slots and two Qt slots (160 KB); the epilogue stages the bf16 tile in the same memory
constexpr int kLdsBytes = kQtBase + 2 * kQtSlot > kBM * kStageRowBytes ? kQtBase + 2 * kQtSlot : kBM * kStageRowBytes;

typedef __attribute__((address_space(3))) void* lds_ptr_t;
typedef float f32x16_t __attribute__((ext_vector_type(16)));

__device__ __forceinline__ f32x16_t mfma32(const u32x4_t& a, const u32x4_t& b, const f32x16_t& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8_t, a), __builtin_bit_cast(bf16x8_t, b), c,
                                                 0, 0, 0);
}
__device__ __forceinline__ u32x4_t lds_read16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

template <int N>
__device__ __forceinline__ void wait_vm() {
  static_assert(N >= 0 && N < 64, "vmcnt range");
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt((N & 15) | ((N >> 4) << 14) | 0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// 16-column groups of Qt are permuted: column n sits at entry pos(n).
__device__ __forceinline__ int qt_pos(int n) { return (n & ~15) | ((n & 15) ^ ((n >> 4) & 15)); }

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
  int bi;
  int64_t mb, nb;
};

// Workgroup id -> (tile, k-split).  Units are ordered split by split, and
// within a split the tile order walks groups of four row tiles column by
// column.  Each XCD (workgroup id mod 8) gets one contiguous run of that
// order: the workgroups on one XCD share P and weight panels in its L2, and
// with a k-split each XCD reads the k-range of one or two splits only.
__device__ __forceinline__ Tile map_unit(const PreArgs& a, int bid, int& ks) {
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
  T.nb = (int64_t)ct * kBN;
  return T;
}

template <bool MASK>
__device__ __forceinline__ void w4_tile(const PreArgs& a, const Tile& T, int ks, char* smem) {
  constexpr int NQ = 8;  // register loads per stage
  const PreOut& O = a.o[T.bi];
  const int w = __builtin_amdgcn_readfirstlane((int)threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int wm = w & 1, wn = w >> 1;
  const int L = l & 31, gL = l >> 5;
  const rsrc_t rP = make_rsrc(O.P, a.rows * O.ldp * 2);
  const rsrc_t rQ = make_rsrc(O.Q, O.qrows * O.ldq * 2);
  const int qcols = (int)min64((int64_t)kBN, O.ldq - T.nb);

  W4_TRACE_TILE(0);
  const int nks_all = (int)((O.kd + 31) / 32);
  const int s0 = ks * a.split_steps;  // even: splits start on a 64-deep stage
  const int nk = max(0, min(nks_all - s0, a.split_steps));
  const int nst = (nk + 1) >> 1;
  const int64_t k0 = (int64_t)s0 * 32;

  // ---- P direct loads: instruction i of wave w fills tile rows 8 (8w + i) .. +7;
  // lane l takes row R = 8 (8w + i) + l / 8, chunk (l % 8) ^ ((R / 2) % 8), which
  // depends on i only through i % 2
  int p_c[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) p_c[h] = (l & 7) ^ ((4 * h + (l >> 4)) & 7);
  const uint32_t p_base = (uint32_t)(((T.mb + 64 * w + (l >> 3)) * O.ldp + k0) * 2);
  const uint32_t p_rows8 = (uint32_t)(16 * O.ldp);  // 8 rows
  // instruction i of this wave's eight for stage st into P slot `slot`
  auto p_issue_one = [&](char* slot, int st, int i) {
    const bool ok = k0 + 8 * p_c[i & 1] + 64 * (int64_t)st < O.kd;
    const uint32_t off = p_base + p_rows8 * (uint32_t)i + 16u * (uint32_t)p_c[i & 1] + 128u * (uint32_t)st;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(slot + (8 * w + i) * 1024), 16,
                                             (int)(ok ? off : kOutOfRange), 0, 0, 0);
  };
  auto p_issue = [&](int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) p_issue_one(smem + (st % kPSlots) * kPSlot, st, i);
  };

  // ---- weight rows: lane (L, gL) loads the 8 elements at columns
  // nb + 8L .. + 7 of rows row0 + i (i < 8), row0 = k0 + 16w + 8gL, from
  // wherever they start (any 2-byte offset)
  const int64_t row0 = k0 + 16 * w + 8 * gL;
  const uint32_t q_base = (uint32_t)(2 * (row0 * O.ldq + T.nb) + 16 * L);
  const uint32_t q_stride = (uint32_t)(128 * O.ldq);  // 64 rows
  const uint32_t q_row = (uint32_t)(2 * O.ldq);        // 1 row
  // the matrix's last element, where a load can lose it (see the top)
  const int64_t q_elems = O.qrows * O.ldq;
  const bool q_tail = (q_elems & 1) == 0;
  const uint32_t q_end = (uint32_t)(2 * q_elems);
  const uint32_t q_last = q_tail ? scalar_elem(O.Q, q_elems - 1) : 0u;
  // Two register sets for the weight rows alternate between stages (rows of
  // stage s + 1 are transposed from one while the rows of stage s + 2 arrive
  // in the other), so no loaded register is ever reused while its load is
  // in flight.
  struct QRegs {
    u32x4_t v[8];
  };
  QRegs qa, qb;
  auto q_issue_row = [&](QRegs& q, int i, int st) {
    const bool ok = row0 + 64 * (int64_t)st + i < O.qrows;
    const uint32_t off = q_base + q_stride * (uint32_t)st + q_row * (uint32_t)i;
    q.v[i] = buf_load16(rQ, ok ? off : kOutOfRange);
  };
  auto q_issue = [&](QRegs& q, int st) {
#pragma unroll
    for (int i = 0; i < 8; ++i) q_issue_row(q, i, st);
  };
  // write offsets into Qt for this lane's 8 columns 8L + e
  const int qt_c = 2 * w + gL;
  const int m7 = (L >> 1) & 7;
  const int qt_w0 = qt_c * 4096 + 16 * (16 * (L >> 1) + ((8 * (L & 1)) ^ (((L >> 1) & 15) & 8)));
  u32x4_t r[8];
  auto q_take_row = [&](const QRegs& q, int i, int st) {
    r[i] = q.v[i];
    // wave-uniform: can a chunk of this wave's rows of stage st reach the
    // last element?  (the furthest element is column nb + 255 of row rmax)
    const int64_t rmax = k0 + 64 * (int64_t)st + 16 * w + 15;
    if (q_tail && rmax * O.ldq + T.nb + 255 >= q_elems - 1) {
      const uint32_t o = q_base + q_stride * (uint32_t)st + q_row * (uint32_t)i;
      const bool lost = (o & 2u) && o < q_end && o + 16u > q_end;
      const int j = (int)((q_end - 2u - o) >> 2);  // dword of the chunk holding the last element
#pragma unroll
      for (int t = 0; t < 4; ++t)
        if (lost && t == j) r[i][t] = q_last;
    }
  };
  // column e of the lane's block: 8 k of column 8L + e, into Qt slot `qt`
  auto q_store_col = [&](int e, char* qt) {
    const int t = e >> 1;
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
    u32x4_t o;
#pragma unroll
    for (int u = 0; u < 4; ++u) o[u] = __builtin_amdgcn_perm(r[2 * u + 1][t], r[2 * u][t], sel);
    if (MASK && 8 * L + e >= qcols) o = zerou4();  // last column tile: columns past the matrix read as zero
    lds_write16(qt + qt_w0 + 16 * (e ^ m7), o);
  };
  auto q_store = [&](const QRegs& q, int st) {
    char* qt = smem + kQtBase + (st & 1) * kQtSlot;
#pragma unroll
    for (int i = 0; i < 8; ++i) q_take_row(q, i, st);
#pragma unroll
    for (int e = 0; e < 8; ++e) q_store_col(e, qt);
  };

  // ---- MFMA operand addresses
  const int xr = (L >> 1) & 7;
  const int y = gL ^ xr;
  const int a_base = 128 * (128 * wm + L);  // + rb * 4096 + 16 (2kk ^ y)
  int b_base[4];
#pragma unroll
  for (int cb = 0; cb < 4; ++cb) b_base[cb] = gL * 4096 + 16 * qt_pos(128 * wn + 32 * cb + L);

  f32x16_t acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;

  auto rd = [&](const char* ps, const char* qs, int kk, u32x4_t(&A)[4], u32x4_t(&B)[4]) {
    const int ao = a_base + 16 * ((2 * kk) ^ y);
#pragma unroll
    for (int rb = 0; rb < 4; ++rb) A[rb] = lds_read16(ps + ao + rb * 4096);
#pragma unroll
    for (int cb = 0; cb < 4; ++cb) B[cb] = lds_read16(qs + b_base[cb] + kk * 8192);
  };
  // MFMAs 2j and 2j + 1 of a k16 block (row block j / 2, column blocks 2 (j % 2) + 0, 1)
  // one of the eight operand reads of k16 block kk: A[i] for i < 4, else B[i - 4]
  auto rd1 = [&](const char* ps, const char* qs, int kk, u32x4_t(&A)[4], u32x4_t(&B)[4], int i) {
    if (i < 4)
      A[i] = lds_read16(ps + a_base + 16 * ((2 * kk) ^ y) + i * 4096);
    else
      B[i - 4] = lds_read16(qs + b_base[i - 4] + kk * 8192);
  };
  // MFMA i of a k16 block: row block i / 4, column block i % 4
  auto mf1 = [&](const u32x4_t(&A)[4], const u32x4_t(&B)[4], int i) {
    acc[i >> 2][i & 3] = mfma32(A[i >> 2], B[i & 3], acc[i >> 2][i & 3]);
  };
  auto fence = [] { __builtin_amdgcn_sched_barrier(0); };
  auto pslot = [&](int st) { return smem + (st % kPSlots) * kPSlot; };
  auto qtslot = [&](int st) { return smem + kQtBase + (st & 1) * kQtSlot; };

  // ---- prologue: P of stages 0-2 requested, the weight rows of stage 0 in
  // Qt, the rows of stage 1 requested, P of stage 0 landed, the operands of
  // the first k16 block of stage 0 read
  u32x4_t A0[4], B0[4], A1[4], B1[4];
  q_issue(qb, 0);
  p_issue(0);
  p_issue(1);
  p_issue(2);
  q_store(qb, 0);
  q_issue(qa, 1);
  wait_vm<16 + NQ>();
  barrier_lds();
  W4_TRACE_TILE(1);
  rd(pslot(0), qtslot(0), 0, A0, B0);

  // Stage s multiplies four k16 blocks (M0..M3, 16 MFMAs each) from two
  // operand register sets; the eight operand reads of block kk + 1 are
  // spread over the first eight MFMAs of block kk, and the other work sits
  // after single MFMAs too (each keeps the matrix core busy for about 32
  // cycles), so the one wave on each SIMD never leaves it idle for long:
  //   M0: the weight rows of stage s + 2 are requested into the register set
  //       stage s - 1 emptied;
  //   M1: the rows of stage s + 1 (requested during stage s - 1) are
  //       transposed into Qt of s + 1;
  //   M2: the last reads of this stage's P slot and Qt;
  //   then P of s + 1 is awaited and the stage's one barrier met;
  //   M3: the first operands of stage s + 1 are read and P of stage s + 3 is
  //       requested into this stage's P slot.
  // sched_barrier fences keep this order.  Requests past the last stage land
  // in slots no later stage reads.  (Spreading the memory requests four to a
  // block instead measured slightly slower.)
  auto stage = [&](int s, const QRegs& qin, QRegs& qout) {
    const char* ps = pslot(s);
    const char* qs = qtslot(s);
    char* qt_next = smem + kQtBase + ((s + 1) & 1) * kQtSlot;
    W4_TRACE(0);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mf1(A0, B0, i);
      fence();
      if (i < 8) rd1(ps, qs, 1, A1, B1, i);
      if ((i & 1) == 0) q_issue_row(qout, i >> 1, s + 2);
      fence();
    }
    W4_TRACE(1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mf1(A1, B1, i);
      fence();
      if (i < 8) rd1(ps, qs, 2, A0, B0, i);
      if (i < 8)
        q_take_row(qin, i, s + 1);
      else
        q_store_col(i - 8, qt_next);
      fence();
    }
    W4_TRACE(2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mf1(A0, B0, i);
      fence();
      if (i < 8) rd1(ps, qs, 3, A1, B1, i);
      fence();
    }
    // P of stage s + 1 must have landed (P of s + 2 and the weight rows of
    // s + 2 may stay in flight); after the barrier every wave has read this
    // stage's P slot and Qt and written Qt of s + 1
    W4_TRACE(3);
    wait_vm<8 + NQ>();
    barrier_lds();
    W4_TRACE(4);
    char* p3 = smem + (s % kPSlots) * kPSlot;  // slot of stage s + 3
    const char* ps1 = pslot(s + 1);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      mf1(A1, B1, i);
      fence();
      if (i < 8)
        rd1(ps1, qt_next, 0, A0, B0, i);
      else
        p_issue_one(p3, s + 3, i - 8);
      fence();
    }
    W4_TRACE(5);
  };
  for (int s = 0; s < nst; s += 2) {
    stage(s, qa, qb);
    if (s + 1 < nst) stage(s + 1, qb, qa);
  }
  W4_TRACE_TILE(2);
  wait_vm<0>();
  barrier_lds();
  W4_TRACE_TILE(4);

  // ------------------------------------------------------------ epilogue --
  // acc[rb][cb] lane l, register 4b + t: row 8b + 4 gL + t of 32-row block
  // 4 wm + rb, column L of 32-column block 4 wn + cb.
  if (a.splits > 1) {
    float* part = O.part + (int64_t)ks * a.rows * O.ldpart;
#pragma unroll
    for (int rb = 0; rb < 4; ++rb)
#pragma unroll
      for (int cb = 0; cb < 4; ++cb)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const int64_t m = T.mb + 128 * wm + 32 * rb + 8 * (e >> 2) + 4 * gL + (e & 3);
          const int64_t n = T.nb + 128 * wn + 32 * cb + L;
          if (m < a.rows && n < O.out_cols) part[m * O.ldpart + n] = acc[rb][cb][e];
        }
    W4_TRACE_TILE(3);
    return;
  }
  const int64_t ldc = O.ldc;
  // Staging: row m of the tile sits at m * kStageRowBytes, shifted by the
  // misalignment d of the output row, which depends only on (T.mb + m) mod 8
  // = (T.mb + 4 gL + e % 4) mod 8 for this lane's registers.
  int sbase[4];
#pragma unroll
  for (int j = 0; j < 4; ++j) {
    const int d = (int)(((T.mb + 4 * gL + j) * ldc + T.nb) & 7);
    sbase[j] = (128 * wm + 4 * gL + j) * kStageRowBytes + 2 * (d + 128 * wn + L);
  }
#pragma unroll
  for (int rb = 0; rb < 4; ++rb)
#pragma unroll
    for (int e = 0; e < 16; ++e) {
      uint16_t* row = reinterpret_cast<uint16_t*>(smem + sbase[e & 3] + (32 * rb + 8 * (e >> 2)) * kStageRowBytes);
#pragma unroll
      for (int cb = 0; cb < 4; ++cb) row[32 * cb] = (uint16_t)f32_to_bf16_rne(acc[rb][cb][e]);
    }
  barrier_lds();
  W4_TRACE_TILE(5);
  // Copy-out: item i = (row i / 33, chunk i % 33), thread t takes items
  // t, t + 256, ... (256 = 7 rows + 25 chunks), so consecutive threads
  // store consecutive 16-byte chunks of a row.  All 33 chunks of a thread
  // are read from LDS first (the accumulators are dead by now), then stored.
  const rsrc_t rC = make_rsrc(O.C, a.rows * ldc * 2);
  const int ncols = (int)min64((int64_t)kBN, O.out_cols - T.nb);
  const int m_first = (int)threadIdx.x / kStageChunks, k_first = (int)threadIdx.x - m_first * kStageChunks;
  u32x4_t chunk[kStageChunks];
  {
    int m = m_first, k = k_first;
#pragma unroll
    for (int it = 0; it < kStageChunks; ++it) {
      chunk[it] = lds_read16(smem + m * kStageRowBytes + 16 * k);
      m += 7;
      k += 25;
      if (k >= kStageChunks) {
        k -= kStageChunks;
        m += 1;
      }
    }
  }
  int m = m_first, k = k_first;
  int64_t rowoff = (T.mb + m) * ldc + T.nb;  // element index of (row, first tile column)
#pragma unroll
  for (int it = 0; it < kStageChunks; ++it) {
    const int d = (int)(rowoff & 7);
    const int n0 = 8 * k - d;
    if (T.mb + m < a.rows && n0 < ncols) {
      const u32x4_t v = chunk[it];
      const int64_t e0 = rowoff + n0;
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
    m += 7;
    k += 25;
    rowoff += 7 * ldc;
    if (k >= kStageChunks) {
      k -= kStageChunks;
      m += 1;
      rowoff += ldc;
    }
  }
  W4_TRACE_TILE(3);
}

__global__ __launch_bounds__(kThreads, 1) void lr_prefill_w4_kernel(const PreArgs a) {
  extern __shared__ __attribute__((aligned(16))) char smem[];
  int ks;
  const Tile T = map_unit(a, (int)blockIdx.x, ks);
  if (a.o[T.bi].ldq - T.nb < kBN)
    w4_tile<true>(a, T, ks, smem);
  else
    w4_tile<false>(a, T, ks, smem);
}

}  // namespace

hipError_t launch_prefill_w4(const PreArgs& args, hipStream_t stream) {
  const int ct = total_col_tiles(args);
  const int grid = ct * args.row_tiles * args.splits;
  if (grid <= 0) return hipSuccess;
  if (args.nb != 8 || args.split_steps % 2 != 0) return hipErrorInvalidValue;
  static std::atomic<uint64_t> attr_done{0};
  const hipError_t e = ensure_dynamic_lds((const void*)lr_prefill_w4_kernel, kLdsBytes, attr_done);
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(lr_prefill_w4_kernel, dim3(grid), dim3(kThreads), kLdsBytes, stream, args);
  return hipGetLastError();
}

}  // namespace lrk
