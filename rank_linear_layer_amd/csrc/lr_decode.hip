// Fused decode kernel (M <= 16): Y = (X . A) . B in ONE launch.
//
// Decode is bound by streaming the two factors from HBM ("LowRankArena
// ...", "Why theoretical FLOPs saved does not equal faster inference" and
// Q3: thin GEMMs, weight streaming and launch overhead dominate; a two-
// kernel low-rank path adds a launch and intermediate-tensor traffic).  This
// kernel therefore reads A and B exactly once, keeps T = X . A off HBM-bound
// round trips (partials live in a small L2/MALL-resident workspace), and
// makes one launch.
//
// Work split (host plan in lr_linear.cpp): the rank is cut into Jw slices of
// 120 columns, K and N into S slices.  Workgroup (js, s):
//   1. GEMM1 partial: T_s[:, js] = X[:, Ks] . A[Ks, js]  (MFMA, split-K);
//      the four waves take alternate 32-row k-tiles; the WG sums them in
//      LDS and publishes the partial with device-coherent stores plus an
//      epoch-stamped flag.
//   2. Prefetch of its first two B tiles is issued before waiting, so the
//      hand-off overlaps B streaming.
//   3. Waits for the S partials of slice js, sums them in fixed order
//      (deterministic), splits T into bf16 hi + lo halves (two MFMAs keep
//      ~16 mantissa bits of T), and computes the partial
//      Y_js[:, Ns] = T[:, js] . B[js, Ns] for its n-slice.
//   4. The last of the Jw workgroups to publish a partial for n-slice s
//      sums the Jw partials in fixed order and writes bf16 Y.
// No floating-point atomics: results are bitwise reproducible.  Counters
// reset themselves and a device-side generation number stamps each launch,
// so no memset is needed between calls.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

constexpr uint32_t kSpinLimit = 1u << 22;

struct RawTile {
  u32x4_t c[8];
};

// Raw chunk loads of one 32-row x 120-column tile (rows rbase + 8g + q).
__device__ __forceinline__ void load_tile_raw(RawTile& t, const uint16_t* __restrict__ base, int64_t rbase,
                                              int64_t nrows, int64_t ld, int64_t colbase, int lane16, int g,
                                              int64_t total) {
#pragma unroll
  for (int q = 0; q < 8; ++q) t.c[q] = load_row_raw(base, rbase + 8 * g + q, nrows, ld, colbase, lane16, total);
}

// Realign + transpose a raw tile into 8 MFMA B-operands (one per column e).
__device__ __forceinline__ void tile_operands(const RawTile& t, u32x4_t op[8], int64_t ld, int64_t colbase,
                                              int lane16, int64_t ncols) {
  u32x4_t seg[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    // rows rbase + 8g + q with rbase, 8g multiples of 8: misalignment (q*ld) mod 8
    const int d = (int)(((int64_t)q * ld + colbase) & 7);
    seg[q] = realign_segment(t.c[q], d, colbase + 8 * lane16, ncols);
  }
  transpose8x8(seg, op);
}

__global__ __launch_bounds__(kDecThreads) void lr_decode_fused_kernel(const DecArgs a) {
  __shared__ float red[kDecWaves][16][kDecJS + 8];
  __shared__ float Ts[16][kDecJS + 8];
  __shared__ uint32_t sh_epoch, sh_old;

  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, np = l & 15, g = l >> 4;

  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProj; ++i)
    if (i < a.nproj && (int)blockIdx.x >= a.p[i].wg_begin) pi = i;
  const DecProj P = a.p[pi];
  const int local = (int)blockIdx.x - P.wg_begin;
  const int js = local / P.S, s = local % P.S;
  const int M = a.M, K = a.K, r = P.r, N = P.N;
  const int64_t totA = (int64_t)K * r, totB = (int64_t)r * N;

  if (tid == 0) sh_epoch = ld_agent_u32(P.ctrl) + 1u;

  // ---------------------------------------------------------- GEMM1 ------
  const int j0 = js * kDecJS;
  const int nk = (K + kDecKT - 1) / kDecKT;
  const int kt_beg = s * P.ktps;
  const int kt_end = min(nk, kt_beg + P.ktps);
  const bool xal = (K & 7) == 0;

  f32x4_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = zero4();

  {
    RawTile t0, t1;
    u32x4_t x0 = zerou4(), x1 = zerou4();
    int kt = kt_beg + w;
    if (kt < kt_end) {
      load_tile_raw(t0, P.A, (int64_t)kt * kDecKT, K, r, j0, np, g, totA);
      x0 = (np < M) ? load_kvec(a.X, np, M, K, (int64_t)kt * kDecKT + 8 * g, K, xal) : zerou4();
    }
    while (kt < kt_end) {
      const int kn = kt + kDecWaves;
      if (kn < kt_end) {
        load_tile_raw(t1, P.A, (int64_t)kn * kDecKT, K, r, j0, np, g, totA);
        x1 = (np < M) ? load_kvec(a.X, np, M, K, (int64_t)kn * kDecKT + 8 * g, K, xal) : zerou4();
      }
      {
        u32x4_t op[8];
        tile_operands(t0, op, r, j0, np, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = mfma_16x16x32(x0, op[e], acc[e]);
      }
      kt = kn;
      if (kt >= kt_end) break;
      const int kn2 = kt + kDecWaves;
      if (kn2 < kt_end) {
        load_tile_raw(t0, P.A, (int64_t)kn2 * kDecKT, K, r, j0, np, g, totA);
        x0 = (np < M) ? load_kvec(a.X, np, M, K, (int64_t)kn2 * kDecKT + 8 * g, K, xal) : zerou4();
      }
      {
        u32x4_t op[8];
        tile_operands(t1, op, r, j0, np, r);
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[e] = mfma_16x16x32(x1, op[e], acc[e]);
      }
      kt = kn2;
    }
  }

  // Prefetch the first two B tiles of this workgroup's n-slice (rows of this
  // wave's 32-row j-tile) before the hand-off.
  const int nn = (N + kDecNT - 1) / kDecNT;
  const int nt_beg = s * P.ntps;
  const int nt_end = min(nn, nt_beg + P.ntps);
  const int64_t jrow0 = (int64_t)j0 + 32 * w;
  const bool wave_has_rows = jrow0 < r && jrow0 < (int64_t)j0 + kDecJS;
  RawTile b0, b1;
  if (wave_has_rows && nt_beg < nt_end)
    load_tile_raw(b0, P.B, jrow0, min64(r, (int64_t)j0 + kDecJS), N, (int64_t)nt_beg * kDecNT, np, g, totB);
  if (wave_has_rows && nt_beg + 1 < nt_end)
    load_tile_raw(b1, P.B, jrow0, min64(r, (int64_t)j0 + kDecJS), N, (int64_t)(nt_beg + 1) * kDecNT, np, g, totB);

  // WG reduction of the four waves' partial T, then publish it.
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[w][4 * g + t][8 * np + e] = acc[e][t];
  __syncthreads();
  {
    float* tp = P.Tpart + (int64_t)(js * P.S + s) * M * kDecJS;
    for (int idx = tid; idx < M * kDecJS; idx += kDecThreads) {
      const int m = idx / kDecJS, jl = idx - m * kDecJS;
      const float v = ((red[0][m][jl] + red[1][m][jl]) + red[2][m][jl]) + red[3][m][jl];
      st_agent_f32(tp + idx, v);
    }
  }
  wait_vmem_all();
  __syncthreads();
  const uint32_t epoch = sh_epoch;
  if (tid == 0) st_agent_u32(P.flags + js * P.S + s, epoch);

  // ----------------------------------------------------- T hand-off ------
  if (w == 0) {
    uint32_t spins = 0;
    while (true) {
      bool ok = true;
      for (int i = l; i < P.S; i += 64) ok = ok && (ld_agent_u32(P.flags + js * P.S + i) == epoch);
      if (__all(ok)) break;
      if (++spins > kSpinLimit) {
        if (l == 0) st_agent_u32(P.ctrl + 2, 1u);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  __syncthreads();
  // Columns kDecJS.. of Ts (read by wave 3's last k-slots) stay zero.
  for (int idx = tid; idx < 16 * (kDecJS + 8); idx += kDecThreads) {
    const int m = idx / (kDecJS + 8), jl = idx - m * (kDecJS + 8);
    float v = 0.f;
    if (m < M && jl < kDecJS) {
      const float* src = P.Tpart + (int64_t)(js * P.S) * M * kDecJS + m * kDecJS + jl;
      for (int ks = 0; ks < P.S; ++ks) v += ld_agent_f32(src + (int64_t)ks * M * kDecJS);
    }
    Ts[m][jl] = v;
  }
  __syncthreads();

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
  const int64_t jrows_end = min64(r, (int64_t)j0 + kDecJS);
  float* yp_base = P.Ypart + ((int64_t)(s * P.Jw + js) * P.ntps) * M * kDecNT;
  auto gemm2_tile = [&](const RawTile& bt, int nt) {
    const int64_t nb = (int64_t)nt * kDecNT;
    f32x4_t y[8];
#pragma unroll
    for (int e = 0; e < 8; ++e) y[e] = zero4();
    if (wave_has_rows) {
      u32x4_t op[8];
      tile_operands(bt, op, N, nb, np, N);
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
    __syncthreads();
    float* yp = yp_base + (int64_t)(nt - nt_beg) * M * kDecNT;
    for (int idx = tid; idx < M * kDecNT; idx += kDecThreads) {
      const int m = idx / kDecNT, nl = idx - m * kDecNT;
      const float v = ((red[0][m][nl] + red[1][m][nl]) + red[2][m][nl]) + red[3][m][nl];
      st_agent_f32(yp + idx, v);
    }
    __syncthreads();
  };
  for (int nt = nt_beg; nt < nt_end; nt += 2) {
    gemm2_tile(b0, nt);
    if (wave_has_rows && nt + 2 < nt_end)
      load_tile_raw(b0, P.B, jrow0, jrows_end, N, (int64_t)(nt + 2) * kDecNT, np, g, totB);
    if (nt + 1 < nt_end) {
      gemm2_tile(b1, nt + 1);
      if (wave_has_rows && nt + 3 < nt_end)
        load_tile_raw(b1, P.B, jrow0, jrows_end, N, (int64_t)(nt + 3) * kDecNT, np, g, totB);
    }
  }

  // ------------------------------------------- final deterministic sum ---
  wait_vmem_all();
  __syncthreads();
  if (tid == 0) sh_old = add_agent_u32(P.ycnt + s, 1u);
  __syncthreads();
  if (sh_old == (uint32_t)(P.Jw - 1)) {
    if (tid == 0) st_agent_u32(P.ycnt + s, 0u);
    const int64_t stride_js = (int64_t)P.ntps * M * kDecNT;
    const float* ys = P.Ypart + (int64_t)s * P.Jw * stride_js;
    const int cnt = (nt_end - nt_beg) * M * kDecNT;
    for (int idx = tid; idx < cnt; idx += kDecThreads) {
      const int ntl = idx / (M * kDecNT);
      const int rem = idx - ntl * M * kDecNT;
      const int m = rem / kDecNT, nl = rem - m * kDecNT;
      const int64_t n = (int64_t)(nt_beg + ntl) * kDecNT + nl;
      float v = 0.f;
      for (int jj = 0; jj < P.Jw; ++jj) v += ld_agent_f32(ys + jj * stride_js + idx);
      if (n < N) P.Y[(int64_t)m * N + n] = (uint16_t)f32_to_bf16_rne(v);
    }
    wait_vmem_all();
    __syncthreads();
    if (tid == 0) {
      const uint32_t old2 = add_agent_u32(P.ctrl + 1, 1u);
      if (old2 == (uint32_t)(P.S - 1)) {
        st_agent_u32(P.ctrl + 1, 0u);
        st_agent_u32(P.ctrl, epoch);
      }
    }
  }
}

hipError_t launch_decode(const DecArgs& args, int grid, hipStream_t stream) {
  hipLaunchKernelGGL(lr_decode_fused_kernel, dim3(grid), dim3(kDecThreads), 0, stream, args);
  return hipGetLastError();
}

int decode_blocks_per_cu() {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lr_decode_fused_kernel, kDecThreads, 0) != hipSuccess) return 0;
  return n;
}

}  // namespace lrk
