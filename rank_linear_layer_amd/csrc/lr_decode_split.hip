// Role-split fused decode kernels (M <= 16): Y = (X . A) . B in one launch,
// with the compute units divided between the two products instead of every
// workgroup taking a share of both.
//
// Decode reads each weight byte once and is bound by HBM ("LowRankArena
// ...", "Why theoretical FLOPs saved does not equal faster inference").  A
// single launch pays its start-up and its end once, but the second product
// needs all of T = X . A: in kernels that give every workgroup a rank slice
// of both factors, the T hand-off sits between the A stream and the B
// stream's use, and the partial Y sums of the rank slices need a second
// hand-off.  Here no partial Y ever leaves a workgroup:
//
//  * T producers: producer j owns rank columns [16 j, 16 j + 16) and
//    computes T[:, those] = X . A[:, those] over all of K, so a T slice is
//    final where it is computed.  It is published as GEMM2's MFMA operand
//    rows, bf16 hi + lo (about fp32 accuracy; for M <= 8 hi and lo share
//    one operand, rows 0-7 and 8-15), into nrep replicas with epoch flags,
//    so that many readers of the same few kilobytes spread over memory
//    channels;
//  * Y producers: each owns 16-column groups of N and computes
//    Y[:, those] = T . B[:, those] over the whole rank.
//
// Three variants:
//  * lr_decode_split_kernel: GA T producers and GB Y producers; a Y
//    producer requests its whole B slab into registers at entry, while the
//    T producers stream A, then waits for the flags, stages one replica of
//    the operand planes in LDS and finishes with one MFMA per step;
//  * lr_decode_splits_kernel (B too large for registers): every workgroup
//    computes Y for a balanced share of the column groups, the first GA
//    after producing their T slice; B streams through registers (and one
//    group through LDS) while each wave keeps its T operands in registers;
//  * lr_decode_splitf_kernel (A-heavy shapes): every workgroup takes an
//    equal share of A's blocks in slice-major order, a slice's first
//    contributor adds the others' fp32 partial tiles and publishes the
//    planes; then Y as in the streaming variant.
//
// Both factors are kept in the MFMA operand block layout of the dense path
// (copied at create): 16 columns x 32 rows per 1 KB block, lane l holding
// rows 32 s + 8 (l / 16) .. + 7 of column l % 16, rows and columns past the
// matrix zero.  Every weight load is one contiguous kilobyte per wave and
// no row alignment reaches the kernel: a misaligned rank or width costs
// only its zero padding.
//
// The epoch of a launch is the generation word ctrl[0] plus one, read by
// every workgroup at entry.  Workgroups count themselves in ctrl[1] once
// they have read the generation; one workgroup (Y producer 0, or the last
// workgroup of the streaming variants) waits for that count and for every
// T flag (each stored after its producer read the generation), then clears
// the count and stores the epoch as the next generation.  No argument
// changes between launches and nothing is cleared from the host, so a
// captured graph can replay a launch.  In the first variant T producers
// have the lowest ids and never wait, so it completes even when not every
// workgroup is resident at once; the other two assume all G workgroups
// are (one per CU; the launcher refuses a grid that does not fit), and
// every spin gives up after spin_limit rounds, raising ctrl[2] and the
// handle's pinned host word.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

namespace {

constexpr int kSpThreads = 512;  // 8 waves
constexpr int kSpWaves = kSpThreads / 64;
constexpr int kSpChunk = 16;     // A blocks in flight per wave at once
#ifndef LR_SPLIT_SLEEP
#define LR_SPLIT_SLEEP 1  // s_sleep units (64 clocks) between flag polls
#endif
constexpr uint32_t kSpOut = 0x7FFFFF00u;  // past every buffer range: loads read 0, stores are dropped

typedef __attribute__((address_space(3))) void* lds_ptr_t;

__device__ __forceinline__ void buf_store_u16(rsrc_t r, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, (int)byte_off, 0, 0);
}

__device__ __forceinline__ void buf_store8_coherent(rsrc_t r, uint32_t byte_off, uint32_t v0, uint32_t v1) {
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  const u32x2_t v = {v0, v1};
  __builtin_amdgcn_raw_buffer_store_b64(v, r, (int)byte_off, 0, kCoherent);
}

// Optional phase timestamps (constant-rate device clock), compiled in only
// with -DLR_DECODE_TRACE: held in scalar registers, stored at the end.
#ifdef LR_DECODE_TRACE
#define SP_TRACE(i) tr[i] = sp_trace_now()
__device__ __forceinline__ uint64_t sp_trace_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : : "memory");
  return t;
}
#else
#define SP_TRACE(i) \
  do {              \
  } while (0)
#endif

// Wave-level: T slice j (lane -> row `row` of the 16 operand rows, columns
// c .. c + 3 of the slice, values v) split into bf16 hi + lo and stored as
// GEMM2's MFMA operand rows in every replica (see P in SplitArgs), then
// every replica's flag of slice j set to `epoch` once the stores are
// acknowledged.
__device__ __forceinline__ void publish_planes(const SplitArgs& a, int j, const float (&v)[4], int row, int c,
                                               uint32_t epoch, int l) {
  const bool packed = a.M <= 8;
  uint32_t hi[2], lo[2];
#pragma unroll
  for (int p = 0; p < 2; ++p) {
    const uint32_t h0 = f32_to_bf16_rne(v[2 * p]), h1 = f32_to_bf16_rne(v[2 * p + 1]);
    hi[p] = h0 | (h1 << 16);
    lo[p] = pack_bf16x2(v[2 * p] - __uint_as_float(h0 << 16), v[2 * p + 1] - __uint_as_float(h1 << 16));
  }
  const bool take_lo = packed && row >= 8;
  const int planes = packed ? 1 : 2;
  const int64_t plane = (int64_t)16 * a.ldp;  // bf16 per plane
  const int64_t rep = plane * planes;         // bf16 per replica
  const rsrc_t rP = make_rsrc(a.P, rep * a.nrep * 2);
  const uint32_t off = (uint32_t)((row * a.ldp + 16 * j + c) * 2);
  for (int q = 0; q < a.nrep; ++q) {
    const uint32_t qo = off + (uint32_t)(q * rep * 2);
    buf_store8_coherent(rP, qo, take_lo ? lo[0] : hi[0], take_lo ? lo[1] : hi[1]);
    if (!packed) buf_store8_coherent(rP, qo + (uint32_t)(plane * 2), lo[0], lo[1]);
  }
  wait_vmem_all();  // the slice is visible before its flags
  if (l < a.nrep)
    buf_store_u32_coherent(make_rsrc(a.flags, (int64_t)a.nrep * a.ldf * 4), (uint32_t)(l * a.ldf + j) * 4u, epoch);
}

// T producer: rank columns [16 j, 16 j + 16) over all of K, eight waves
// splitting the k-steps, then the slice published and flagged.
template <bool XAL>
__device__ __forceinline__ void t_producer(const SplitArgs& a, int j, uint32_t epoch, float (*red)[256], uint64_t* tr) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int nk = a.nkA;
  const int per = (nk + kSpWaves - 1) / kSpWaves;
  const int s0 = min(nk, w * per), s1 = min(nk, s0 + per);
  const rsrc_t rA = make_rsrc(a.Asw + (int64_t)j * nk * 512, (int64_t)nk * 1024);
  const rsrc_t rX = make_rsrc(a.X, (int64_t)a.M * a.K * 2);
  // MFMA A operand of lane l: X row m = l % 16 (rows >= M read as zero),
  // columns 32 s + 8 (l / 16) .. + 7; unaligned rows are loaded as the two
  // aligned chunks around them and shifted per lane
  const int m = l & 15;
  const int64_t xrow = (int64_t)m * a.K;
  const int d = (int)(xrow & 7);
  f32x4_t acc = zero4();
  for (int c0 = s0; c0 < s1; c0 += kSpChunk) {
    u32x4_t wv[kSpChunk], xl[kSpChunk], xh[kSpChunk];
#pragma unroll
    for (int i = 0; i < kSpChunk; ++i) {
      const int s = c0 + i;
      wv[i] = buf_load16(rA, s < s1 ? (uint32_t)(s * 1024 + l * 16) : kSpOut);
      const int64_t e = xrow + 32 * s + 8 * (l >> 4);
      if (XAL) {
        xl[i] = buf_load16(rX, (uint32_t)(e * 2));
      } else {
        xl[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16));
        xh[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16 + 16));
      }
    }
#pragma unroll
    for (int i = 0; i < kSpChunk; ++i) {
      // columns >= K are cleared (they hold the next row, and 0 * NaN is not 0)
      const u32x4_t x = mask_cols(XAL ? xl[i] : realign_lane(xl[i], xh[i], d), 32 * (c0 + i) + 8 * (l >> 4), a.K);
      acc = mfma_16x16x32(m < a.M ? x : zerou4(), wv[i], acc);
    }
  }
  SP_TRACE(1);
  // acc lane l, register t: row 4 (l / 16) + t, column l % 16
#pragma unroll
  for (int t = 0; t < 4; ++t) red[w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc[t];
  barrier_lds();
  SP_TRACE(2);
  if (w == 0) {
    // lane -> row l / 4, columns 4 (l % 4) .. + 3 of the slice; the waves'
    // partials summed in wave order, then split into bf16 hi + lo and
    // stored as GEMM2's MFMA operand rows (see P in SplitArgs): with
    // M <= 8, rows 0-7 of plane 0 hold hi and rows 8-15 lo of T rows 0-7;
    // otherwise plane 0 holds hi and plane 1 lo of T rows 0-15.  Rows of T
    // >= M are exactly zero (so are their X rows), which clears whatever a
    // call with a larger M left there.
    const bool packed = a.M <= 8;
    const int row = l >> 2, c = (l & 3) * 4;
    const int trow = packed ? (row & 7) : row;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float s = 0.f;
#pragma unroll
      for (int q = 0; q < kSpWaves; ++q) s += red[q][trow * 16 + c + i];
      v[i] = s;
    }
    publish_planes(a, j, v, row, c, epoch, l);
  }
  SP_TRACE(3);
}

// Wave 0 spins until the 32-bit words [first, first + count) of `r` all
// equal `want` (and, when `count_too`, ctrl[1] equals `count_want`), with
// device-coherent loads.  Gives up after spin_limit rounds and raises the
// timeout flags.  The flag words are compared with want ^ stall_xor (see
// SplitArgs).
__device__ __forceinline__ void spin_until(const SplitArgs& a, rsrc_t r, int first, int count, uint32_t want,
                                           bool count_too, uint32_t count_want, int lane) {
  const rsrc_t rC = make_rsrc(a.ctrl, 8);
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
    for (int i = lane; i < count; i += 64) {
      const uint32_t off = (uint32_t)(first + i) * 4u;
      ok = ok && (buf_load_u32_coherent(r, off) == (want ^ a.stall_xor));
    }
    if (count_too && lane == 0) ok = ok && (buf_load_u32_coherent(rC, 4u) == count_want);
    if (__all(ok)) break;
    if (++spins > a.spin_limit) {
      if (lane == 0) raise_stall(a.ctrl, a.err);
      break;
    }
    __builtin_amdgcn_s_sleep(LR_SPLIT_SLEEP);
  }
}

// Y producer b: column groups b * gpw .. + gpw - 1, the waves of a group
// splitting the rank's k-steps; NB = B blocks held per wave.  `tlds`
// receives T's operand planes (whole kilobytes).
template <int NB>
__device__ __forceinline__ void y_producer(const SplitArgs& a, int b, uint32_t gen, uint32_t epoch, float (*red)[256],
                                           char* tlds, uint64_t* tr) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int wpg = kSpWaves / a.gpw;  // waves per column group
  const int gi = w / wpg, sub = w - gi * wpg;
  const int64_t g = (int64_t)b * a.gpw + gi;
  const int nk = a.nkB;
  const int per = (nk + wpg - 1) / wpg;
  const int s0 = min(nk, sub * per), s1 = min(nk, s0 + per);
  const bool gok = g < a.GN;
  const rsrc_t rB = make_rsrc(a.Bsw, (int64_t)a.GN * nk * 1024);
  const uint32_t gbase = (uint32_t)(g * nk * 1024);

  // count this producer in (no return value: nothing waits for it).  The
  // increment takes its operand from an empty asm statement that reads the
  // generation, so it cannot be issued before the generation load returned.
  if (tid == 0) {
    uint32_t one = 1u;
    asm volatile("" : "+v"(one) : "s"(gen));
    (void)add_agent_u32(a.ctrl + 1, one);
  }

  // the whole B slab of this wave, requested at once
  u32x4_t bv[NB];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const int s = s0 + i;
    bv[i] = buf_load16(rB, (gok && s < s1) ? gbase + (uint32_t)(s * 1024 + l * 16) : kSpOut);
  }
  SP_TRACE(4);

  // T hand-off: this producer reads replica b % nrep of T and of the T
  // flags (every replica holds all of T), so that the producers' reads of
  // the same few kilobytes spread over nrep copies in different memory
  // channels.  Y producer 0 also waits for the count of Y producers: with
  // every T flag and every Y producer in, every workgroup of the launch has
  // read the generation, and it stores the next one.
  const int q = b % a.nrep;
  const bool packed = a.M <= 8;
  const int64_t plane = (int64_t)16 * a.ldp;
  const int64_t pbytes = plane * (packed ? 1 : 2) * 2;
  const rsrc_t rP = make_rsrc(a.P + (int64_t)q * plane * (packed ? 1 : 2), pbytes);
  const rsrc_t rF = make_rsrc(a.flags + (int64_t)q * a.ldf, (int64_t)a.GA * 4);
  const int nchunk = (int)((pbytes + 1023) / 1024);
  if (w == 0) spin_until(a, rF, 0, a.GA, epoch, b == 0, (uint32_t)a.GB, l);
  if (b == 0 && tid == 0) {
    st_agent_u32(a.ctrl + 1, 0u);
    st_agent_u32(a.ctrl, epoch);
  }
  barrier_lds();
  SP_TRACE(5);
  // T's operand planes into LDS: device-coherent direct loads, one kilobyte
  // per wave instruction, each workgroup starting at a different kilobyte
  const int c0 = (b * 5) % nchunk;
  for (int c = w; c < nchunk; c += kSpWaves) {
    const int cc = c0 + c < nchunk ? c0 + c : c0 + c - nchunk;
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rP, (lds_ptr_t)(tlds + cc * 1024), 16, cc * 1024 + l * 16, 0, 0, kCoherent);
  }
  wait_vmem_all();
  barrier_lds();
  SP_TRACE(11);

  // GEMM2: lane l, step s reads its operand (row l % 16, columns
  // 32 s + 8 (l / 16) .. + 7) straight from the planes.  With M <= 8 one
  // MFMA per step (output rows m and m + 8 add up to Y row m), otherwise
  // hi then lo.  Steps past this wave's range meet zero B blocks.
  const uint16_t* prow = reinterpret_cast<const uint16_t*>(tlds) + (l & 15) * a.ldp + 8 * (l >> 4);
  f32x4_t acc = zero4();
  if (packed) {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = min(s0 + i, nk - 1);
      acc = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(prow + 32 * s), bv[i], acc);
    }
  } else {
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      const int s = min(s0 + i, nk - 1);
      acc = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(prow + 32 * s), bv[i], acc);
      acc = mfma_16x16x32(*reinterpret_cast<const u32x4_t*>(prow + plane + 32 * s), bv[i], acc);
    }
  }
  SP_TRACE(7);
#pragma unroll
  for (int t = 0; t < 4; ++t) red[w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc[t];
  barrier_lds();
  SP_TRACE(8);
  for (int idx = tid; idx < a.gpw * 256; idx += kSpThreads) {
    const int gq = idx >> 8, e = idx & 255;
    const int row = e >> 4, col = e & 15;
    float sum = 0.f;
    for (int q2 = 0; q2 < wpg; ++q2) sum += red[gq * wpg + q2][e];
    if (packed) {
      float sum_lo = 0.f;
      if (row < 8)
        for (int q2 = 0; q2 < wpg; ++q2) sum_lo += red[gq * wpg + q2][e + 128];
      sum += sum_lo;
    }
    const int64_t n = 16 * ((int64_t)b * a.gpw + gq) + col;
    if (row < a.M && n < a.N) a.Y[(int64_t)row * a.N + n] = (uint16_t)f32_to_bf16_rne(sum);
  }
  SP_TRACE(9);
}

// Count this workgroup in (ctrl[1]; no return value, so nothing waits for
// it).  The increment takes its operand from an empty asm statement that
// reads the generation, so it cannot be issued before that load returned.
__device__ __forceinline__ void count_in(const SplitArgs& a, uint32_t gen) {
  if (threadIdx.x == 0) {
    uint32_t one = 1u;
    asm volatile("" : "+v"(one) : "s"(gen));
    (void)add_agent_u32(a.ctrl + 1, one);
  }
}

// The B blocks of column group g for this wave's k-steps [s0, s1) (zeros
// when !ok or past s1).
template <int NB>
__device__ __forceinline__ void load_group(u32x4_t (&buf)[NB], rsrc_t rB, int64_t g, int nk, int s0, int s1, bool ok,
                                           int l) {
  const uint32_t base = (uint32_t)(g * nk * 1024) + (uint32_t)(l * 16);
#pragma unroll
  for (int i = 0; i < NB; ++i)
    buf[i] = buf_load16(rB, (ok && s0 + i < s1) ? base + (uint32_t)((s0 + i) * 1024) : kSpOut);
}

// The first two column groups' B blocks of this wave, requested ahead of
// the rest of the Y work (y_stream refills the same buffers); a third
// group (g0 + 2) goes straight into this wave's LDS region `glds` (NB
// kilobytes per wave).
template <int NB>
struct YBufs {
  u32x4_t b0[NB], b1[NB];
};
template <int NB>
__device__ __forceinline__ void y_prefetch(const SplitArgs& a, int g0, int g1, YBufs<NB>& yb, char* glds) {
  const int w = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
  const int l = threadIdx.x & 63;
  const int nk = a.nkB;
  const int per = (nk + kSpWaves - 1) / kSpWaves;
  const int s0 = min(nk, w * per), s1 = min(nk, s0 + per);
  const rsrc_t rB = make_rsrc(a.Bsw, (int64_t)a.GN * nk * 1024);
  load_group<NB>(yb.b0, rB, g0, nk, s0, s1, g0 < g1, l);
  load_group<NB>(yb.b1, rB, g0 + 1, nk, s0, s1, g0 + 1 < g1, l);
  const bool ok = g0 + 2 < g1;
  const uint32_t base = (uint32_t)((int64_t)(g0 + 2) * nk * 1024) + (uint32_t)(l * 16);
#pragma unroll
  for (int i = 0; i < NB; ++i)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(rB, (lds_ptr_t)(glds + (w * NB + i) * 1024), 16,
                                             (ok && s0 + i < s1) ? (int)(base + (uint32_t)((s0 + i) * 1024)) : (int)kSpOut,
                                             0, 0, 0);
}

// Y work of the streaming variants: column groups [g0, g1), each over the
// whole rank, the eight waves splitting its k-steps.  A wave loads its T
// operands once and keeps them in registers for every group.  The group
// staged in LDS is multiplied first, then the others stream through the
// two register buffers, each refilled as soon as its MFMAs are issued;
// each group's eight partials are summed in LDS (two buffers, one barrier
// per group) and stored as bf16.  `writer`: this workgroup also waits for
// every workgroup's count and stores the next generation.
template <int NB, bool TWO>
__device__ __forceinline__ void y_stream(const SplitArgs& a, int wg, int g0, int g1, uint32_t epoch, bool writer,
                                         float (*red)[kSpWaves][256], uint64_t* tr, YBufs<NB>& yb, const char* glds) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int nk = a.nkB;
  const int per = (nk + kSpWaves - 1) / kSpWaves;
  const int s0 = min(nk, w * per), s1 = min(nk, s0 + per);
  const rsrc_t rB = make_rsrc(a.Bsw, (int64_t)a.GN * nk * 1024);
  u32x4_t(&b0)[NB] = yb.b0;
  u32x4_t(&b1)[NB] = yb.b1;
  SP_TRACE(4);

  // every T slice published (device-coherent flags of replica wg % nrep)
  const int q = wg % a.nrep;
  constexpr bool packed = !TWO;  // TWO: M > 8, hi and lo in two planes
  const int64_t plane = (int64_t)16 * a.ldp;
  if (w == 0) spin_until(a, make_rsrc(a.flags + (int64_t)q * a.ldf, (int64_t)a.GA * 4), 0, a.GA, epoch, writer,
                         (uint32_t)a.G, l);
  if (writer && tid == 0) {
    st_agent_u32(a.ctrl + 1, 0u);
    st_agent_u32(a.ctrl, epoch);
  }
  barrier_lds();
  SP_TRACE(5);
  // this wave's T operands: lane l, step s -> plane row l % 16, columns
  // 32 s + 8 (l / 16) .. + 7.  Rows that hold only zeros for this M are not
  // fetched (out-of-range offsets read as zero).
  const int m = l & 15;
  const bool row_used = packed ? (m & 7) < a.M : m < a.M;
  const rsrc_t rP = make_rsrc(a.P + (int64_t)q * plane * (packed ? 1 : 2), plane * (packed ? 1 : 2) * 2);
  const uint32_t pbase = (uint32_t)((m * a.ldp + 8 * (l >> 4)) * 2);
  u32x4_t t0[NB], t1[TWO ? NB : 1];
#pragma unroll
  for (int i = 0; i < NB; ++i) {
    const bool ok = row_used && s0 + i < s1;
    const uint32_t off = pbase + (uint32_t)((s0 + i) * 64);
    t0[i] = __builtin_bit_cast(u32x4_t, buf_load16_coherent(rP, ok ? off : kSpOut));
    if constexpr (TWO) t1[i] = __builtin_bit_cast(u32x4_t, buf_load16_coherent(rP, ok ? off + (uint32_t)(plane * 2) : kSpOut));
  }
  SP_TRACE(11);

  const rsrc_t rY = make_rsrc(a.Y, (int64_t)a.M * a.N * 2);
  int buf = 0;
  auto mma = [&](const u32x4_t(&bv)[NB]) {
    f32x4_t acc = zero4();
#pragma unroll
    for (int i = 0; i < NB; ++i) {
      acc = mfma_16x16x32(t0[i], bv[i], acc);
      if constexpr (TWO) acc = mfma_16x16x32(t1[i], bv[i], acc);
    }
    return acc;
  };
  // sum group g's partials and store them (stores past M, N or g1 are dropped)
  auto finish = [&](const f32x4_t& acc, int g) {
#pragma unroll
    for (int t = 0; t < 4; ++t) red[buf][w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc[t];
    barrier_lds();
    if (tid < 256) {
      const int row = tid >> 4, col = tid & 15;
      float sum = 0.f;
#pragma unroll
      for (int v = 0; v < kSpWaves; ++v) sum += red[buf][v][tid];
      if (packed && row < 8) {
        float lo = 0.f;
#pragma unroll
        for (int v = 0; v < kSpWaves; ++v) lo += red[buf][v][tid + 128];
        sum += lo;
      }
      const int64_t n = 16 * (int64_t)g + col;
      const bool ok = g < g1 && row < a.M && n < a.N;
      buf_store_u16(rY, ok ? (uint32_t)((row * (int64_t)a.N + n) * 2) : kSpOut, f32_to_bf16_rne(sum));
    }
    buf ^= 1;
  };
  // the group staged in LDS first (its loads were the last prefetched, so
  // waiting for everything in flight costs nothing more), then the rest
  // through the registers: groups g0, g0 + 1, g0 + 3, g0 + 4, ...
  const bool in_lds = g0 + 2 < g1;
  if (in_lds) {
    wait_vmem_all();
    u32x4_t bl[NB];
#pragma unroll
    for (int i = 0; i < NB; ++i) bl[i] = *reinterpret_cast<const u32x4_t*>(glds + (w * NB + i) * 1024 + l * 16);
    finish(mma(bl), g0 + 2);
  }
  const int nreg = g1 - g0 - (in_lds ? 1 : 0);
  auto gmap = [&](int k) { return g0 + k + (in_lds && k >= 2 ? 1 : 0); };
  // two groups in flight: a buffer is refilled as soon as its MFMAs are
  // issued, before the group's partials are summed
  for (int k = 0; k < nreg; k += 2) {
    const f32x4_t acc0 = mma(b0);
    load_group<NB>(b0, rB, gmap(k + 2), nk, s0, s1, k + 2 < nreg, l);
    finish(acc0, gmap(k));
    const f32x4_t acc1 = mma(b1);
    load_group<NB>(b1, rB, gmap(k + 3), nk, s0, s1, k + 3 < nreg, l);
    finish(acc1, k + 1 < nreg ? gmap(k + 1) : g1);
  }
  SP_TRACE(9);
}

// First contributor (workgroup) of the flat block range that holds block b:
// the largest w with floor(w TB / G) <= b.
__device__ __forceinline__ int flat_owner(int64_t b, int64_t TB, int G) {
  return (int)(((b + 1) * G + TB - 1) / TB) - 1;
}

// T work of the flat variant: workgroup wg takes the A blocks
// [wg TB / G, (wg + 1) TB / G) of the operand block layout, which is in
// slice-major order (TB = GA ceil(K/32) blocks), so its range covers parts
// of at most two rank slices (GA <= G).  The eight waves split the range;
// a block of the first slice accumulates into acc0, of the second into
// acc1 (two predicated MFMAs per block, no branch).  Per slice segment:
// the slice's first contributor (lowest id) owns it: it waits for the
// other contributors' fp32 partials, adds them to its own in contributor
// order and publishes the operand planes; every other contributor
// publishes its partial (device-coherent, with an epoch flag) and never
// waits.  Wave 0 handles the first segment, wave 1 the second.
template <bool XAL>
__device__ __forceinline__ void t_flat(const SplitArgs& a, int wg, uint32_t epoch, float (*red)[kSpWaves][256],
                                       uint64_t* tr) {
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int nk = a.nkA;
  const int64_t TB = (int64_t)a.GA * nk;
  const int64_t b_lo = (int64_t)wg * TB / a.G, b_hi = (int64_t)(wg + 1) * TB / a.G;
  const int j0 = (int)(b_lo / nk);
  const int64_t split_at = (int64_t)(j0 + 1) * nk;  // first block of the second slice
  const int64_t pw = (b_hi - b_lo + kSpWaves - 1) / kSpWaves;
  const int64_t w_lo = min64(b_hi, b_lo + w * pw), w_hi = min64(b_hi, w_lo + pw);
  const rsrc_t rA = make_rsrc(a.Asw, TB * 1024);
  const rsrc_t rX = make_rsrc(a.X, (int64_t)a.M * a.K * 2);
  const int m = l & 15;
  const int64_t xrow = (int64_t)m * a.K;
  const int d = (int)(xrow & 7);
  f32x4_t acc0 = zero4(), acc1 = zero4();
  for (int64_t c0 = w_lo; c0 < w_hi; c0 += kSpChunk) {
    u32x4_t wv[kSpChunk], xl[kSpChunk], xh[kSpChunk];
#pragma unroll
    for (int i = 0; i < kSpChunk; ++i) {
      const int64_t b = c0 + i;
      wv[i] = buf_load16(rA, b < w_hi ? (uint32_t)(b * 1024 + l * 16) : kSpOut);
      const int64_t s = b - (b >= split_at ? split_at : split_at - nk);  // k-step within its slice
      const int64_t e = xrow + 32 * s + 8 * (l >> 4);
      if (XAL) {
        xl[i] = buf_load16(rX, (uint32_t)(e * 2));
      } else {
        xl[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16));
        xh[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16 + 16));
      }
    }
#pragma unroll
    for (int i = 0; i < kSpChunk; ++i) {
      const int64_t b = c0 + i;
      const int64_t s = b - (b >= split_at ? split_at : split_at - nk);
      const u32x4_t x0 = mask_cols(XAL ? xl[i] : realign_lane(xl[i], xh[i], d), 32 * s + 8 * (l >> 4), a.K);
      const u32x4_t x = m < a.M ? x0 : zerou4();
      const bool second = b >= split_at;
      acc0 = mfma_16x16x32(second ? zerou4() : x, wv[i], acc0);
      acc1 = mfma_16x16x32(second ? x : zerou4(), wv[i], acc1);
    }
  }
  SP_TRACE(1);
#pragma unroll
  for (int t = 0; t < 4; ++t) {
    red[0][w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc0[t];
    red[1][w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc1[t];
  }
  barrier_lds();
  SP_TRACE(2);
  const int nseg = b_hi > split_at ? 2 : 1;
  if (w < nseg) {
    const int seg = w;
    const int j = j0 + seg;
    const int64_t s_beg = (int64_t)j * nk;                 // the slice's blocks
    const int64_t s_end = s_beg + nk;
    const int first = flat_owner(s_beg, TB, a.G), last = flat_owner(s_end - 1, TB, a.G);
    const bool packed = a.M <= 8;
    const int row = l >> 2, c = (l & 3) * 4;
    const int trow = packed ? (row & 7) : row;
    float v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      float sum = 0.f;
#pragma unroll
      for (int q = 0; q < kSpWaves; ++q) sum += red[seg][q][trow * 16 + c + i];
      v[i] = sum;
    }
    // partials: [GA][maxc] tiles of 16 x 16 fp32 (rows as T rows), flags [GA][maxc]
    const rsrc_t rPart = make_rsrc(a.part, (int64_t)a.GA * a.maxc * 1024);
    const rsrc_t rPF = make_rsrc(a.pflags, (int64_t)a.GA * a.maxc * 4);
    const int ci = wg - first;
    if (ci > 0) {
      // not the owner: publish the partial (T rows 0..15, this lane's row
      // `row` and columns c..c+3) and its flag
      f32x4_t pv;
      for (int i = 0; i < 4; ++i) {
        float sum = 0.f;
#pragma unroll
        for (int q = 0; q < kSpWaves; ++q) sum += red[seg][q][row * 16 + c + i];
        pv[i] = sum;
      }
      buf_store16_coherent(rPart, (uint32_t)(((int64_t)j * a.maxc + ci) * 1024 + (row * 16 + c) * 4), pv);
      wait_vmem_all();
      if (l == 0) buf_store_u32_coherent(rPF, (uint32_t)(j * a.maxc + ci) * 4u, epoch);
    } else {
      // the owner: add the other contributors' partials in order
      const int n = last - first + 1;
      if (n > 1) {
        uint32_t spins = 0;
        while (true) {
          bool ok = true;
          for (int q = 1 + l; q < n; q += 64) ok = ok && (buf_load_u32_coherent(rPF, (uint32_t)(j * a.maxc + q) * 4u) == epoch);
          if (__all(ok)) break;
          if (++spins > a.spin_limit) {
            if (l == 0) raise_stall(a.ctrl, a.err);
            break;
          }
          __builtin_amdgcn_s_sleep(LR_SPLIT_SLEEP);
        }
        for (int q = 1; q < n; ++q) {
          const f32x4_t pv = buf_load16_coherent(rPart, (uint32_t)(((int64_t)j * a.maxc + q) * 1024 + (trow * 16 + c) * 4));
#pragma unroll
          for (int i = 0; i < 4; ++i) v[i] += pv[i];
        }
      }
      publish_planes(a, j, v, row, c, epoch, l);
    }
  }
  SP_TRACE(3);
}

}  // namespace

template <int NB, bool XAL>
__global__ __launch_bounds__(kSpThreads) void lr_decode_split_kernel(const SplitArgs a) {
  __shared__ float red[kSpWaves][256];
  extern __shared__ __align__(16) char sp_tlds[];  // Y producers: T's operand planes
  uint64_t tr[16] = {};
  SP_TRACE(15);
  const uint32_t gen = __builtin_amdgcn_readfirstlane(ld_agent_u32(a.ctrl));
  const uint32_t epoch = gen + 1u == 0u ? 1u : gen + 1u;
  SP_TRACE(0);
  const int wg = blockIdx.x;
  if (wg < a.GA)
    t_producer<XAL>(a, wg, epoch, red, tr);
  else
    y_producer<NB>(a, wg - a.GA, gen, epoch, red, sp_tlds, tr);
#ifdef LR_DECODE_TRACE
  if (a.trace && threadIdx.x == 0)
    for (int i = 0; i < 16; ++i) a.trace[blockIdx.x * 16 + i] = tr[i];
#else
  (void)tr;
#endif
}

int split_blocks_per_wave(const SplitArgs& a) {
  const int wpg = kSpWaves / a.gpw;
  return (a.nkB + wpg - 1) / wpg;
}

// Streaming variant: every workgroup computes Y for its column groups; the
// first GA also produce T first (and take fewer groups).
template <int NB, bool XAL, bool TWO>
__global__ __launch_bounds__(kSpThreads) void lr_decode_splits_kernel(const SplitArgs a) {
  __shared__ float red[2][kSpWaves][256];
  extern __shared__ __align__(16) char sp_glds[];  // one column group's B blocks, NB KB per wave
  uint64_t tr[16] = {};
  SP_TRACE(15);
  const uint32_t gen = __builtin_amdgcn_readfirstlane(ld_agent_u32(a.ctrl));
  const uint32_t epoch = gen + 1u == 0u ? 1u : gen + 1u;
  SP_TRACE(0);
  count_in(a, gen);
  const int wg = blockIdx.x;
  int g0, g1;
  if (wg < a.GA) {
    g0 = wg * a.nt;
    g1 = g0 + a.nt;
  } else {
    const int y = wg - a.GA, gy = a.G - a.GA;
    const int rest = a.GN - a.GA * a.nt;
    g0 = a.GA * a.nt + (int)((int64_t)y * rest / gy);
    g1 = a.GA * a.nt + (int)((int64_t)(y + 1) * rest / gy);
  }
  g1 = min(g1, a.GN);
  YBufs<NB> yb;
  if (wg < a.GA) t_producer<XAL>(a, wg, epoch, red[0], tr);
  y_prefetch<NB>(a, g0, g1, yb, sp_glds);
  y_stream<NB, TWO>(a, wg, g0, g1, epoch, wg == a.G - 1, red, tr, yb, sp_glds);
#ifdef LR_DECODE_TRACE
  if (a.trace && threadIdx.x == 0)
    for (int i = 0; i < 16; ++i) a.trace[blockIdx.x * 16 + i] = tr[i];
#else
  (void)tr;
#endif
}

template <int NB, bool XAL, bool TWO>
hipError_t launch_splits_variant(const SplitArgs& a, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  static std::atomic<uint64_t> occ{0};
  hipError_t e = ensure_dynamic_lds((const void*)lr_decode_splits_kernel<NB, XAL, TWO>, kSpWaves * NB * 1024, attr_done);
  if (e == hipSuccess)
    e = check_coresident((const void*)lr_decode_splits_kernel<NB, XAL, TWO>, kSpThreads, (size_t)kSpWaves * NB * 1024, a.G, occ);
  if (e != hipSuccess || a.check_only) return e;
  hipLaunchKernelGGL((lr_decode_splits_kernel<NB, XAL, TWO>), dim3((unsigned)a.G), dim3(kSpThreads),
                     (size_t)kSpWaves * NB * 1024, stream, a);
  return hipGetLastError();
}

// Flat variant: every workgroup takes an equal share of A (in slice-major
// block order) and then an equal share of Y's column groups.
template <int NB, bool XAL, bool TWO>
__global__ __launch_bounds__(kSpThreads) void lr_decode_splitf_kernel(const SplitArgs a) {
  __shared__ float red[2][kSpWaves][256];
  extern __shared__ __align__(16) char sp_glds[];  // one column group's B blocks, NB KB per wave
  uint64_t tr[16] = {};
  SP_TRACE(15);
  const uint32_t gen = __builtin_amdgcn_readfirstlane(ld_agent_u32(a.ctrl));
  const uint32_t epoch = gen + 1u == 0u ? 1u : gen + 1u;
  SP_TRACE(0);
  count_in(a, gen);
  const int wg = blockIdx.x;
  const int g0 = (int)((int64_t)wg * a.GN / a.G), g1 = (int)((int64_t)(wg + 1) * a.GN / a.G);
  // B is requested only once this workgroup's share of A is in and its T
  // work published: requested earlier, it slows the A stream that every
  // slice waits for
  t_flat<XAL>(a, wg, epoch, red, tr);
  YBufs<NB> yb;
  y_prefetch<NB>(a, g0, g1, yb, sp_glds);
  y_stream<NB, TWO>(a, wg, g0, g1, epoch, wg == a.G - 1, red, tr, yb, sp_glds);
#ifdef LR_DECODE_TRACE
  if (a.trace && threadIdx.x == 0)
    for (int i = 0; i < 16; ++i) a.trace[blockIdx.x * 16 + i] = tr[i];
#else
  (void)tr;
#endif
}

template <int NB, bool XAL, bool TWO>
hipError_t launch_splitf_variant(const SplitArgs& a, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  static std::atomic<uint64_t> occ{0};
  hipError_t e = ensure_dynamic_lds((const void*)lr_decode_splitf_kernel<NB, XAL, TWO>, kSpWaves * NB * 1024, attr_done);
  if (e == hipSuccess)
    e = check_coresident((const void*)lr_decode_splitf_kernel<NB, XAL, TWO>, kSpThreads, (size_t)kSpWaves * NB * 1024, a.G, occ);
  if (e != hipSuccess || a.check_only) return e;
  hipLaunchKernelGGL((lr_decode_splitf_kernel<NB, XAL, TWO>), dim3((unsigned)a.G), dim3(kSpThreads),
                     (size_t)kSpWaves * NB * 1024, stream, a);
  return hipGetLastError();
}

template <int NB, bool XAL>
hipError_t launch_split_variant(const SplitArgs& a, size_t lds, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  static std::atomic<uint64_t> occ{0};
  hipError_t e = ensure_dynamic_lds((const void*)lr_decode_split_kernel<NB, XAL>, (int)kSplitMaxTBytes, attr_done);
  if (e == hipSuccess)
    e = check_coresident((const void*)lr_decode_split_kernel<NB, XAL>, kSpThreads, lds, (int64_t)a.GA + a.GB, occ);
  if (e != hipSuccess || a.check_only) return e;
  hipLaunchKernelGGL((lr_decode_split_kernel<NB, XAL>), dim3((unsigned)(a.GA + a.GB)), dim3(kSpThreads), lds, stream, a);
  return hipGetLastError();
}

hipError_t launch_decode_split(const SplitArgs& a, hipStream_t stream) {
  if (a.stream_y == 2) {
    // flat variant: GA <= G (a workgroup's share of A spans at most two
    // slices), partial tiles for maxc contributors per slice
    const int per = (a.nkB + kSpWaves - 1) / kSpWaves;
    const int64_t TB = (int64_t)a.GA * a.nkA;
    if (a.M < 1 || a.M > 16 || a.GA < 1 || a.G < a.GA || TB < a.G || TB * 1024 >= ((int64_t)1 << 31) || a.ldp < 32 * a.nkB ||
        a.ldp % 8 != 0 || 16 * a.GA > a.ldp || a.nrep < 1 || a.nrep > 64 || a.ldf < a.GA || per > kSplitMaxBlocks ||
        (a.M > 8 && per > 8) || a.maxc < 1 || !a.part || !a.pflags)
      return hipErrorInvalidValue;
    // every slice's contributors fit the partial table: a slice of nkA
    // blocks meets at most ceil(nkA / R) + 1 ranges of length >= R (>= 1:
    // TB >= G, so no workgroup's share is empty)
    const int64_t R = TB / a.G;
    if ((a.nkA + R - 1) / R + 1 > a.maxc) return hipErrorInvalidValue;
    const bool xal = (a.K & 7) == 0;
    if (a.M > 8) {
      if (per <= 4) return xal ? launch_splitf_variant<4, true, true>(a, stream) : launch_splitf_variant<4, false, true>(a, stream);
      return xal ? launch_splitf_variant<8, true, true>(a, stream) : launch_splitf_variant<8, false, true>(a, stream);
    }
    if (per <= 4) return xal ? launch_splitf_variant<4, true, false>(a, stream) : launch_splitf_variant<4, false, false>(a, stream);
    if (per <= 8) return xal ? launch_splitf_variant<8, true, false>(a, stream) : launch_splitf_variant<8, false, false>(a, stream);
    if (per <= 12)
      return xal ? launch_splitf_variant<12, true, false>(a, stream) : launch_splitf_variant<12, false, false>(a, stream);
    return xal ? launch_splitf_variant<16, true, false>(a, stream) : launch_splitf_variant<16, false, false>(a, stream);
  }
  if (a.stream_y) {
    // streaming variant: G workgroups, the first GA also T producers with nt
    // groups each; every wave of a workgroup holds at most kSplitMaxBlocks
    // B blocks of a group (twice) and as many T operands (twice for M > 8)
    const int per = (a.nkB + kSpWaves - 1) / kSpWaves;
    if (a.M < 1 || a.M > 16 || a.GA < 1 || a.G < a.GA || a.G < 1 || a.nt < 0 || (a.G > a.GA && (int64_t)a.GA * a.nt > a.GN) ||
        (a.G == a.GA && (int64_t)a.GA * a.nt < a.GN) || a.ldp < 32 * a.nkB || a.ldp % 8 != 0 || 16 * a.GA > a.ldp ||
        a.nrep < 1 || a.nrep > 64 || a.ldf < a.GA || per > kSplitMaxBlocks || (a.M > 8 && per > 8))
      return hipErrorInvalidValue;
    const bool xal = (a.K & 7) == 0;
    if (a.M > 8) {
      if (per <= 4) return xal ? launch_splits_variant<4, true, true>(a, stream) : launch_splits_variant<4, false, true>(a, stream);
      return xal ? launch_splits_variant<8, true, true>(a, stream) : launch_splits_variant<8, false, true>(a, stream);
    }
    if (per <= 4) return xal ? launch_splits_variant<4, true, false>(a, stream) : launch_splits_variant<4, false, false>(a, stream);
    if (per <= 8) return xal ? launch_splits_variant<8, true, false>(a, stream) : launch_splits_variant<8, false, false>(a, stream);
    if (per <= 12)
      return xal ? launch_splits_variant<12, true, false>(a, stream) : launch_splits_variant<12, false, false>(a, stream);
    return xal ? launch_splits_variant<16, true, false>(a, stream) : launch_splits_variant<16, false, false>(a, stream);
  }
  if (a.M < 1 || a.M > 16 || a.GA < 1 || a.GB < 1 || !(a.gpw == 1 || a.gpw == 2 || a.gpw == 4 || a.gpw == 8))
    return hipErrorInvalidValue;
  if ((int64_t)a.GB * a.gpw < a.GN || a.ldp < 32 * a.nkB || a.ldp % 8 != 0 || 16 * a.GA > a.ldp || a.nrep < 1 ||
      a.nrep > 64 || a.ldf < a.GA)
    return hipErrorInvalidValue;
  const size_t lds = (size_t)((16 * a.ldp * 2 * (a.M <= 8 ? 1 : 2) + 1023) / 1024) * 1024;
  if (lds > (size_t)kSplitMaxTBytes) return hipErrorInvalidValue;
  const int nb = split_blocks_per_wave(a);
  const bool xal = (a.K & 7) == 0;
  if (nb <= 4) return xal ? launch_split_variant<4, true>(a, lds, stream) : launch_split_variant<4, false>(a, lds, stream);
  if (nb <= 8) return xal ? launch_split_variant<8, true>(a, lds, stream) : launch_split_variant<8, false>(a, lds, stream);
  if (nb <= kSplitMaxBlocks)
    return xal ? launch_split_variant<kSplitMaxBlocks, true>(a, lds, stream)
               : launch_split_variant<kSplitMaxBlocks, false>(a, lds, stream);
  return hipErrorInvalidValue;
}

}  // namespace lrk
