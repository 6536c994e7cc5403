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
//   3. T hand-off: the partial is published with device-coherent stores; the
//      last of the S workgroups of slice js to arrive sums the S partials in
//      fixed order and publishes T_js with an epoch-stamped flag, which the
//      others poll;
//   4. GEMM2 partial Y_js[:, Ns] = T_js . B[js, Ns] with T split into bf16
//      hi + lo halves (two MFMAs keep ~16 mantissa bits of T);
//   5. the last of the Jw workgroups to publish a partial for n-slice s sums
//      the Jw partials in fixed order and writes bf16 Y.
// No floating-point atomics: results are bitwise reproducible.  Counters
// reset themselves and a device-side generation number stamps each launch,
// so no memset is needed between calls.
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

// out[v] = sum over p < npart (in order) of the float4 at
// base + p * pstride + (tid + 256 v) * 16, for vector indices < nvec.
template <int V>
__device__ __forceinline__ void sum_partials(rsrc_t ws, uint32_t base, uint32_t pstride, int npart, int nvec,
                                             int tid, f32x4_t out[V]) {
#pragma unroll
  for (int v = 0; v < V; ++v) out[v] = zero4();
  for (int p0 = 0; p0 < npart; p0 += 8) {
    f32x4_t t[8][V];
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) {
        const int vi = tid + kDecThreads * v;
        const bool ok = (p0 + u < npart) && (vi < nvec);
        const uint32_t off = ok ? base + (uint32_t)(p0 + u) * pstride + (uint32_t)vi * 16u : base;
        const f32x4_t x = buf_load16_coherent(ws, off);
        t[u][v] = ok ? x : zero4();
      }
#pragma unroll
    for (int u = 0; u < 8; ++u)
#pragma unroll
      for (int v = 0; v < V; ++v) out[v] += t[u][v];
  }
}

__global__ __launch_bounds__(kDecThreads) void lr_decode_fused_kernel(const DecArgs a) {
  DEC_TRACE_ENTRY();
  __shared__ float red[kDecWaves][16][kDecJS + 8];
  __shared__ float Ts[16][kDecJS + 8];
  __shared__ uint32_t sh_epoch, sh_old;

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
  if (tid == 0) sh_epoch = ld_agent_u32(P.ctrl) + 1u;

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
  RawTile ta[kDecABuf], b0, b1;
  u32x4_t xa[kDecABuf];
  const int kt0 = kt_beg + w;
#pragma unroll
  for (int i = 0; i < kDecABuf; ++i) {
    const int k = kt0 + kDecWaves * i;
    load_tile_raw_if(ta[i], rA, (int64_t)k * kDecKT, r, j0, np, g, k < kt_end);
    xa[i] = load_kvec(rX, np, K, (int64_t)k * kDecKT + 8 * g, K, xal);
  }
  if (nt_beg < nt_end) load_tile_raw(b0, rB, jrow0, N, (int64_t)nt_beg * kDecNT, np, g);
  if (nt_beg + 1 < nt_end) load_tile_raw(b1, rB, jrow0, N, (int64_t)(nt_beg + 1) * kDecNT, np, g);

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

  // WG reduction of the four waves' partial T; publish it (float4 rows of
  // kDecJS floats, M rows).
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w][4 * g + t][8 * np + e] = acc[e][t];
  barrier_lds();
  DEC_TRACE(1);
  constexpr int kV4 = kDecJS / 4;  // float4 per row of a slice
  const int nvecT = M * kV4;
  const uint32_t slice_bytes = (uint32_t)(M * kDecJS * 4);
  for (int vi = tid; vi < nvecT; vi += kDecThreads) {
    const int m = vi / kV4, c = (vi - m * kV4) * 4;
    f32x4_t v;
#pragma unroll
    for (int i = 0; i < 4; ++i) v[i] = ((red[0][m][c + i] + red[1][m][c + i]) + red[2][m][c + i]) + red[3][m][c + i];
    buf_store16_coherent(rW, P.off_tpart + (uint32_t)(js * P.S + s) * slice_bytes + (uint32_t)vi * 16u, v);
  }
  wait_vmem_all();
  barrier_lds();
  DEC_TRACE(2);
  const uint32_t epoch = sh_epoch;
  if (tid == 0) sh_old = add_agent_u32(P.tcnt + js, 1u);
  barrier_lds();
  DEC_TRACE(3);

  // ----------------------------------------------------- T hand-off ------
  if (sh_old == (uint32_t)(P.S - 1)) {
    // Last arriver: reduce the S partials of slice js in order, publish T_js.
    if (tid == 0) st_agent_u32(P.tcnt + js, 0u);
    f32x4_t sum[1];
    for (int vbase = 0; vbase < nvecT; vbase += kDecThreads) {
      sum_partials<1>(rW, P.off_tpart + (uint32_t)(js * P.S) * slice_bytes + (uint32_t)vbase * 16u, slice_bytes,
                      P.S, nvecT - vbase, tid, sum);
      const int vi = vbase + tid;
      if (vi < nvecT) {
        buf_store16_coherent(rW, P.off_tfin + (uint32_t)js * slice_bytes + (uint32_t)vi * 16u, sum[0]);
        const int m = vi / kV4, c = (vi - m * kV4) * 4;
#pragma unroll
        for (int i = 0; i < 4; ++i) Ts[m][c + i] = sum[0][i];
      }
    }
    wait_vmem_all();
    barrier_lds();
    if (tid == 0) st_agent_u32(P.tflag + js, epoch);
  } else {
    if (w == 0) {
      uint32_t spins = 0;
      while (true) {
        const bool ok = ld_agent_u32(P.tflag + js) == (epoch ^ P.stall_xor);
        if (ok) break;
        if (++spins > P.spin_limit) {
          if (l == 0) raise_stall(P.ctrl, P.err);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
    }
    barrier_lds();
    for (int vi = tid; vi < nvecT; vi += kDecThreads) {
      const f32x4_t v = buf_load16_coherent(rW, P.off_tfin + (uint32_t)js * slice_bytes + (uint32_t)vi * 16u);
      const int m = vi / kV4, c = (vi - m * kV4) * 4;
#pragma unroll
      for (int i = 0; i < 4; ++i) Ts[m][c + i] = v[i];
    }
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
  const uint32_t ypart_wg = P.off_ypart + (uint32_t)((s * P.Jw + js) * P.ntps) * (uint32_t)(M * kDecNT * 4);
  // One n-tile: its partial is stored only when `ok` (a tile past the end of
  // the slice is computed on zeros and its stores are dropped).
  auto gemm2_tile = [&](const RawTile& bt, int nt, bool ok) {
    const int64_t nb = (int64_t)nt * kDecNT;
    f32x4_t y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = zero4();
    {
      u32x4_t op[8];
      tile_operands(bt, op, jrow0, g, jrow_end, N, nb, np, N);
#pragma unroll
      for (int e = 0; e < 8; ++e) {
        y[e] = mfma_16x16x32(thi, op[e], y[e]);
        y[e] = mfma_16x16x32(tlo, op[e], y[e]);
      }
    }
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int t = 0; t < 4; ++t) red[w][4 * g + t][8 * np + e] = y[e][t];
    barrier_lds();
    const uint32_t yp = ypart_wg + (uint32_t)(nt - nt_beg) * (uint32_t)(M * kDecNT * 4);
    for (int vi = tid; vi < M * (kDecNT / 4); vi += kDecThreads) {
      const int m = vi / (kDecNT / 4), c = (vi - m * (kDecNT / 4)) * 4;
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) v[i] = ((red[0][m][c + i] + red[1][m][c + i]) + red[2][m][c + i]) + red[3][m][c + i];
      buf_store16_coherent(rW, off_if(yp + (uint32_t)vi * 16u, ok), v);
    }
    barrier_lds();
  };
  // Tiles in pairs with no branch around a load or store: the next tile of
  // each buffer is requested (or replaced by zeros) right after its use.
  for (int nt = nt_beg; nt < nt_end; nt += 2) {
    gemm2_tile(b0, nt, true);
    load_tile_raw_if(b0, rB, jrow0, N, (int64_t)(nt + 2) * kDecNT, np, g, nt + 2 < nt_end);
    gemm2_tile(b1, nt + 1, nt + 1 < nt_end);
    load_tile_raw_if(b1, rB, jrow0, N, (int64_t)(nt + 3) * kDecNT, np, g, nt + 3 < nt_end);
  }

  // ------------------------------------------- final deterministic sum ---
  DEC_TRACE(5);
  wait_vmem_all();
  barrier_lds();
  if (tid == 0) sh_old = add_agent_u32(P.ycnt + s, 1u);
  barrier_lds();
  DEC_TRACE(6);
  if (sh_old == (uint32_t)(P.Jw - 1)) {
    if (tid == 0) st_agent_u32(P.ycnt + s, 0u);
    const uint32_t stride_js = (uint32_t)P.ntps * (uint32_t)(M * kDecNT * 4);
    const uint32_t ys = P.off_ypart + (uint32_t)(s * P.Jw) * stride_js;
    const int nvecY = (nt_end - nt_beg) * M * (kDecNT / 4);
    f32x4_t sum[2];
    for (int vbase = 0; vbase < nvecY; vbase += 2 * kDecThreads) {
      sum_partials<2>(rW, ys + (uint32_t)vbase * 16u, stride_js, P.Jw, nvecY - vbase, tid, sum);
#pragma unroll
      for (int v = 0; v < 2; ++v) {
        const int vi = vbase + tid + kDecThreads * v;
        if (vi >= nvecY) continue;
        const int ntl = vi / (M * (kDecNT / 4));
        const int rem = vi - ntl * M * (kDecNT / 4);
        const int m = rem / (kDecNT / 4), c = (rem - m * (kDecNT / 4)) * 4;
        const int64_t n0 = (int64_t)(nt_beg + ntl) * kDecNT + c;
#pragma unroll
        for (int i = 0; i < 4; ++i)
          if (n0 + i < N) P.Y[(int64_t)m * N + n0 + i] = (uint16_t)f32_to_bf16_rne(sum[v][i]);
      }
    }
    wait_vmem_all();
    barrier_lds();
    if (tid == 0) {
      const uint32_t old2 = add_agent_u32(P.ctrl + 1, 1u);
      if (old2 == (uint32_t)(P.S - 1)) {
        st_agent_u32(P.ctrl + 1, 0u);
        st_agent_u32(P.ctrl, epoch);
      }
    }
  }
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
