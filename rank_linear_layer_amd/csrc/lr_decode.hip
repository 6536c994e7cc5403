// Fused decode kernel (M <= 16): Y = (X . A) . B in ONE launch.
//
// Decode is bound by streaming the two factors from HBM ("LowRankArena
// ...", "Why theoretical FLOPs saved does not equal faster inference" and
// Q3: thin GEMMs, weight streaming and launch overhead dominate; a two-
// kernel low-rank path adds a launch and intermediate-tensor traffic).  This
// kernel therefore reads A and B exactly once, never sends T through HBM
// round trips (partials live in a small L2/MALL-resident workspace), and
// makes one launch.
//
// Work split (host plan in lr_validate.h): the rank is cut into Jw slices
// of 120 columns, K and N into S slices.  Workgroup (js, s):
//   1. issues the loads of its A tiles and of its first two B tiles at once,
//      so all of its HBM traffic is in flight from the start;
//   2. GEMM1 partial T_s[:, js] = X[:, Ks] . A[Ks, js] (MFMA); the four waves
//      take alternate 32-row k-tiles and are summed in LDS;
//   3. T hand-off: the partial is published as epoch-tagged exchange words
//      (lr_device.h); every one of the S workgroups of slice js polls the S
//      partials and sums them in fixed order (one hop, no last arriver);
//   4. GEMM2 partial Y_js[:, Ns] = T_js . B[js, Ns] with T split into bf16
//      hi + lo halves (two MFMAs keep ~16 mantissa bits of T), published as
//      exchange words;
//   5. the Jw workgroups of n-slice s each poll their 1/Jw share of it in the
//      Jw partials, sum it in fixed order and write bf16 Y.
// No atomics: results are bitwise reproducible.  A device-side generation
// number stamps each launch (workgroup 0 advances it at its end), so no
// memset is needed between calls and a captured graph can replay them.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

// Optional phase timestamps (constant-rate device clock), compiled in only
// with -DLR_DECODE_TRACE; used to see where a launch spends its time.  They
// are held in scalar registers and stored when the kernel ends, so that no
// trace store sits in the vector-memory counter that the phases wait on.
#ifdef LR_DECODE_TRACE
__device__ __forceinline__ uint64_t dec_trace_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : : "memory");
  return t;
}
#define DEC_TRACE_ENTRY()     \
  uint64_t trace_t_[16] = {}; \
  trace_t_[15] = dec_trace_now()
#define DEC_TRACE_ENTRY_STORE() do { } while (0)
#define DEC_TRACE(i) trace_t_[i] = dec_trace_now()
#define DEC_TRACE_FLUSH()                                                                        \
  do {                                                                                           \
    if (a.trace && tid == 0)                                                                     \
      for (int i_ = 0; i_ < 16; ++i_) a.trace[blockIdx.x * kDecTracePoints + i_] = trace_t_[i_]; \
  } while (0)
#else
#define DEC_TRACE_ENTRY() do { } while (0)
#define DEC_TRACE_ENTRY_STORE() do { } while (0)
#define DEC_TRACE(i) \
  do {               \
  } while (0)
#define DEC_TRACE_FLUSH() do { } while (0)
#endif

struct RawTile {
  u32x4_t c[8];
};

// Offsets with bit 31 set lie past the end of every buffer range (matrices
// and the workspace are below 2 GiB): such a load returns zeros and such a
// store is dropped, without touching memory.  Loads and stores that depend
// on a condition use this instead of a branch: at the join of a branch
// around memory instructions the compiler must assume the shorter queue and
// waits for every request in flight, which collapses double buffering.
__device__ __forceinline__ uint32_t off_if(uint32_t off, bool ok) { return off | ((uint32_t)!ok << 31); }

__device__ __forceinline__ void load_tile_raw_if(RawTile& t, rsrc_t r, int64_t rbase, int64_t ld, int64_t colbase,
                                                 int lane16, int g, bool ok) {
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int64_t c0 = ((rbase + 8 * g + q) * ld + colbase) >> 3;
    t.c[q] = buf_load16(r, off_if((uint32_t)((c0 + lane16) * 16), ok));
  }
}

// Raw chunk loads of one 32-row x 120-column tile (rows rbase + 8g + q).
__device__ __forceinline__ void load_tile_raw(RawTile& t, rsrc_t r, int64_t rbase, int64_t ld, int64_t colbase,
                                              int lane16, int g) {
#pragma unroll
  for (int q = 0; q < 8; ++q) t.c[q] = load_row_raw(r, rbase + 8 * g + q, ld, colbase, lane16);
}

// Realign + transpose a raw tile into 8 MFMA B-operands (one per column e).
// Rows >= row_end are zeroed.
__device__ __forceinline__ void tile_operands(const RawTile& t, u32x4_t op[8], int64_t rbase, int g,
                                              int64_t row_end, int64_t ld, int64_t colbase, int lane16,
                                              int64_t ncols) {
  u32x4_t seg[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    // rbase and 8g are multiples of 8, so the misalignment is (q * ld + colbase) mod 8
    const int d = (int)(((int64_t)q * ld + colbase) & 7);
    seg[q] = realign_segment(t.c[q], d, colbase + 8 * lane16, ncols, rbase + 8 * g + q < row_end);
  }
  transpose8x8(seg, op);
}

__global__ __launch_bounds__(kDecThreads) void lr_decode_fused_kernel(const DecArgs a) {
  DEC_TRACE_ENTRY();
  __shared__ float red[kDecWaves][16][kDecJS + 8];
  __shared__ float red2[kDecWaves][16][kDecJS + 8];  // the second n-tile of a GEMM2 pair
  __shared__ float Ts[16][kDecJS + 8];
  __shared__ uint32_t sh_epoch;

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l = tid & 63, np = l & 15, g = l >> 4;

  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProj; ++i)
    if (i < a.nproj && (int)blockIdx.x >= a.p[i].wg_begin) pi = i;
  const DecProj P = a.p[pi];
  const int local = (int)blockIdx.x - P.wg_begin;
  // Workgroup -> (rank slice, K/N slice).  With a verified round-robin XCD
  // dispatch, each XCD takes a contiguous run of the rank-slice-major order,
  // so adjacent rank slices (which share the 128-byte lines around their
  // boundaries in A) are fetched into the same L2.  Any bijection is
  // correct; this one only saves HBM traffic.
  int js, s;
  if (P.xcd_local) {
    const int G = P.Jw * P.S;
    const int x = local & 7, slot = local >> 3;
    const int p = x * (G >> 3) + min(x, G & 7) + slot;
    js = p / P.S;
    s = p - js * P.S;
  } else {
    js = local / P.S;
    s = local - js * P.S;
  }
  const int M = a.M, K = a.K, r = P.r, N = P.N;

  const rsrc_t rA = make_rsrc(P.A, (int64_t)K * r * 2);
  const rsrc_t rB = make_rsrc(P.B, (int64_t)r * N * 2);
  const rsrc_t rX = make_rsrc(a.X, (int64_t)M * K * 2);
  const rsrc_t rW = make_rsrc(P.ws, P.ws_bytes);

  DEC_TRACE(0);
  DEC_TRACE_ENTRY_STORE();
  if (tid == 0) {
    const uint32_t gen = ld_agent_u32(P.ctrl);
    sh_epoch = gen + 1u == 0u ? 1u : gen + 1u;  // 0 is the value of fresh memory
  }

  // ------------------------------------------------ issue all loads -----
  const int j0 = js * kDecJS;
  const int nk = (K + kDecKT - 1) / kDecKT;
  const int kt_beg = s * P.ktps;
  const int kt_end = min(nk, kt_beg + P.ktps);
  const bool xal = (K & 7) == 0;

  const int nn = (N + kDecNT - 1) / kDecNT;
  const int nt_beg = s * P.ntps;
  const int nt_end = min(nn, nt_beg + P.ntps);
  const int64_t jrow0 = (int64_t)j0 + 32 * w;
  const int64_t jrow_end = min64(r, (int64_t)j0 + kDecJS);

  // This wave's k-tiles are kt0, kt0 + 4, ...; a ring of kDecABuf of them is
  // in flight from the start (with the X segments they meet), and each is
  // requested again right after its use, with no branch around a load.
  constexpr int kDecABuf = 4;
  // B tiles in flight per wave (3 or 4 measured slower: the extra requests
  // compete with A's stream)
  constexpr int kDecBBuf = 2;
  RawTile ta[kDecABuf], tb[kDecBBuf];
  u32x4_t xa[kDecABuf];
  const int kt0 = kt_beg + w;
#pragma unroll
  for (int i = 0; i < kDecABuf; ++i) {
    const int k = kt0 + kDecWaves * i;
    load_tile_raw_if(ta[i], rA, (int64_t)k * kDecKT, r, j0, np, g, k < kt_end);
    xa[i] = load_kvec(rX, np, K, (int64_t)k * kDecKT + 8 * g, K, xal);
  }
#pragma unroll
  for (int i = 0; i < kDecBBuf; ++i)
    load_tile_raw_if(tb[i], rB, jrow0, N, (int64_t)(nt_beg + i) * kDecNT, np, g, nt_beg + i < nt_end);

  // ---------------------------------------------------------- GEMM1 ------
  f32x4_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = zero4();
  for (int base = kt0; base < kt_end; base += kDecWaves * kDecABuf) {
#pragma unroll
    for (int i = 0; i < kDecABuf; ++i) {
      const int k = base + kDecWaves * i;
      if (k < kt_end) {
        u32x4_t op[8];
        tile_operands(ta[i], op, (int64_t)k * kDecKT, g, K, r, j0, np, r);
        const u32x4_t xm = kvec_mask(xa[i], (int64_t)k * kDecKT + 8 * g, K);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = mfma_16x16x32(xm, op[e], acc[e]);
      }
      const int kn = k + kDecWaves * kDecABuf;
      load_tile_raw_if(ta[i], rA, (int64_t)kn * kDecKT, r, j0, np, g, kn < kt_end);
      xa[i] = load_kvec(rX, np, K, (int64_t)kn * kDecKT + 8 * g, K, xal);
    }
  }

  // WG reduction of the four waves' partial T, published as exchange words
  // (lr_device.h): row m of the slice is words [kHP m, kHP m + kHP).
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w][4 * g + t][8 * np + e] = acc[e][t];
  barrier_lds();
  DEC_TRACE(1);
  constexpr int kHP = kDecJS / 2;  // exchange words per row of a slice
  const int nqT = M * kHP;
  const uint32_t blkT = (uint32_t)(M * kHP * 16);
  const uint32_t tgrp = P.off_tpart + (uint32_t)(js * P.S) * blkT;
  const uint32_t epoch = sh_epoch;
  const float tagf = __uint_as_float(epoch);
  for (int q = tid; q < nqT; q += kDecThreads) {
    const int m = q / kHP, c = 2 * (q - m * kHP);
    const float v0 = ((red[0][m][c] + red[1][m][c]) + red[2][m][c]) + red[3][m][c];
    const float v1 = ((red[0][m][c + 1] + red[1][m][c + 1]) + red[2][m][c + 1]) + red[3][m][c + 1];
    xstore_coherent(rW, tgrp + (uint32_t)s * blkT + (uint32_t)q * 16u, v0, v1, tagf);
  }
  DEC_TRACE(2);
  DEC_TRACE(3);

  // ----------------------------------------------------- T hand-off ------
  // Every member of slice js polls the S partials and sums them in order
  // s = 0..S-1 (bitwise the same T_js in every member); one hop, no counter
  // and no last arriver.  The stall test flag changes the epoch this wait
  // looks for.
  for (int q = tid; q < nqT; q += kDecThreads) {
    float s0, s1;
    xpoll_sum(rW, tgrp, blkT, P.S, (uint32_t)q * 16u, epoch ^ P.stall_xor, P.spin_limit, P.ctrl, P.err, s0, s1);
    const int m = q / kHP, c = 2 * (q - m * kHP);
    Ts[m][c] = s0;
    Ts[m][c + 1] = s1;
  }
  // rows >= M and columns >= kDecJS of Ts are zero (read as operands)
  for (int idx = tid; idx < 16 * (kDecJS + 8); idx += kDecThreads) {
    const int m = idx / (kDecJS + 8), jl = idx - m * (kDecJS + 8);
    if (m >= M || jl >= kDecJS) Ts[m][jl] = 0.f;
  }
  barrier_lds();
  DEC_TRACE(4);

  // bf16 hi/lo split of this wave's 32 rank rows: lane (i = np, g) holds
  // T[i][32w + 8g + q], q = 0..7.
  u32x4_t thi, tlo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float t0v = Ts[np][32 * w + 8 * g + 2 * p];
    const float t1v = Ts[np][32 * w + 8 * g + 2 * p + 1];
    const uint32_t h0 = f32_to_bf16_rne(t0v), h1 = f32_to_bf16_rne(t1v);
    thi[p] = h0 | (h1 << 16);
    tlo[p] = pack_bf16x2(t0v - __uint_as_float(h0 << 16), t1v - __uint_as_float(h1 << 16));
  }

  // ---------------------------------------------------------- GEMM2 ------
  // Y partial of n-tile nt: [M][kDecNT] values as exchange words
  const uint32_t ytile_b = (uint32_t)(M * kDecNT * 8);
  const uint32_t ypart_wg = P.off_ypart + (uint32_t)((s * P.Jw + js) * P.ntps) * ytile_b;
  // A pair of n-tiles nt, nt + 1: both products, one LDS reduction over the
  // four waves' rank rows (two barriers per pair), and the partials' stores;
  // tile nt + 1's are dropped when `ok1` is false (past the slice: computed
  // on zeros).
  auto gemm2_pair = [&](int nt, bool ok1) {
    f32x4_t y0[8], y1[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y0[e] = zero4();
      y1[e] = zero4();
    }
    {
      u32x4_t op[8];
      tile_operands(tb[0], op, jrow0, g, jrow_end, N, (int64_t)nt * kDecNT, np, N);
      // the buffer is free once its operands are formed: request its next tile
      load_tile_raw_if(tb[0], rB, jrow0, N, (int64_t)(nt + 2) * kDecNT, np, g, nt + 2 < nt_end);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y0[e] = mfma_16x16x32(thi, op[e], y0[e]);
        y0[e] = mfma_16x16x32(tlo, op[e], y0[e]);
      }
    }
    {
      u32x4_t op[8];
      tile_operands(tb[1], op, jrow0, g, jrow_end, N, (int64_t)(nt + 1) * kDecNT, np, N);
      load_tile_raw_if(tb[1], rB, jrow0, N, (int64_t)(nt + 3) * kDecNT, np, g, nt + 3 < nt_end);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y1[e] = mfma_16x16x32(thi, op[e], y1[e]);
        y1[e] = mfma_16x16x32(tlo, op[e], y1[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int t = 0; t < 4; ++t) {
        red[w][4 * g + t][8 * np + e] = y0[e][t];
        red2[w][4 * g + t][8 * np + e] = y1[e][t];
      }
    barrier_lds();
    const int nv = M * (kDecNT / 4);
    for (int v2 = tid; v2 < 2 * nv; v2 += kDecThreads) {
      const int h = v2 >= nv ? 1 : 0, vi = v2 - h * nv;
      float(*rr)[16][kDecJS + 8] = h ? red2 : red;
      const int m = vi / (kDecNT / 4), c = (vi - m * (kDecNT / 4)) * 4;
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ((rr[0][m][c + i] + rr[1][m][c + i]) + rr[2][m][c + i]) + rr[3][m][c + i];
      const uint32_t yp = ypart_wg + (uint32_t)(nt + h - nt_beg) * ytile_b;
      const bool ok = h == 0 || ok1;
      xstore_coherent(rW, off_if(yp + (uint32_t)vi * 32u, ok), v[0], v[1], tagf);
      xstore_coherent(rW, off_if(yp + (uint32_t)vi * 32u + 16u, ok), v[2], v[3], tagf);
    }
    barrier_lds();
  };
  // Pairs of tiles with no branch around a load or store: the next tile of
  // each buffer is requested (or replaced by zeros) right after its use.
  for (int nt = nt_beg; nt < nt_end; nt += 2) gemm2_pair(nt, nt + 1 < nt_end);

  // ---------------------------------- Y reduce-scatter over the Jw slices --
  // Member js of n-slice s polls its 1/Jw share of the n-slice's exchange
  // words in the Jw partials (word q at byte 16 q of a partial), sums them
  // in order js' = 0..Jw-1 and writes bf16 Y.
  DEC_TRACE(5);
  const int nty = nt_end - nt_beg;
  if (nty > 0) {
    const uint32_t stride_js = (uint32_t)P.ntps * ytile_b;
    const uint32_t ys = P.off_ypart + (uint32_t)(s * P.Jw) * stride_js;
    const int qtot = nty * M * (kDecNT / 2);
    const int share = (qtot + P.Jw - 1) / P.Jw;
    const int q_lo = js * share, q_hi = min(qtot, q_lo + share);
    for (int q = q_lo + tid; q < q_hi; q += kDecThreads) {
      float s0, s1;
      xpoll_sum(rW, ys, stride_js, P.Jw, (uint32_t)q * 16u, epoch, P.spin_limit, P.ctrl, P.err, s0, s1);
      const int vi = q >> 1;  // float4 of [nty][M][kDecNT / 4]
      const int ntl = vi / (M * (kDecNT / 4));
      const int rem = vi - ntl * M * (kDecNT / 4);
      const int m = rem / (kDecNT / 4), c = (rem - m * (kDecNT / 4)) * 4 + 2 * (q & 1);
      const int64_t n0 = (int64_t)(nt_beg + ntl) * kDecNT + c;
      if (n0 < N) P.Y[(int64_t)m * N + n0] = (uint16_t)f32_to_bf16_rne(s0);
      if (n0 + 1 < N) P.Y[(int64_t)m * N + n0 + 1] = (uint16_t)f32_to_bf16_rne(s1);
    }
  }
  DEC_TRACE(6);
  // The next launch's generation.  Workgroup 0 is (js, s) = (0, 0); its
  // thread 0 polled word 0 of n-slice 0 from every rank slice, each of which
  // followed the T partials of all its K slices, so every workgroup of the
  // launch has read the word by now.
  if (local == 0 && tid == 0) st_agent_u32(P.ctrl, epoch);
  DEC_TRACE(7);
  DEC_TRACE_FLUSH();
}

hipError_t launch_decode(const DecArgs& args, int grid, hipStream_t stream) {
  static std::atomic<uint64_t> occ{0};
  const hipError_t e = check_coresident((const void*)lr_decode_fused_kernel, kDecThreads, 0, grid, occ);
  if (e != hipSuccess || args.check_only) return e;
  hipLaunchKernelGGL(lr_decode_fused_kernel, dim3(grid), dim3(kDecThreads), 0, stream, args);
  return hipGetLastError();
}

int decode_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lr_decode_fused_kernel, kDecThreads, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace lrk
