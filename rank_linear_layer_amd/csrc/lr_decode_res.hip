// LDS-resident fused decode kernel (M <= 16): Y = (X . A) . B, one launch.
//
// Same method as lr_decode.hip, for shapes whose per-workgroup slabs fit in
// LDS (the plan checks this; every other shape takes lr_decode.hip).
// Decode is bound by reading A and B from HBM once ("LowRankArena ...",
// "Why theoretical FLOPs saved does not equal faster inference").  Every
// byte a workgroup needs goes straight into LDS (buffer_load ... lds): no
// VGPRs are tied up by loads in flight.  A (with X) is requested first and
// alone, so that GEMM1 and the T hand-off can start as early as possible;
// B is requested once the T partial is published and streams in during the
// hand-off.  Adjacent rank slices sit on one XCD, so the 128-byte lines that
// straddle two slices of a misaligned A row are fetched once into that
// XCD's L2.
//
// Wave roles keep the in-order vector-memory counter from coupling phases:
// waves 0-1 load X and A and publish the T partial, waves 2-3 load B.
//
// Work split: the rank is cut into Jw slices of JS <= 128 columns (Jw a
// multiple of 8), K and N into S slices.  Workgroup (js, s):
//   GEMM1  T_s[:, js] = X[:, Ks] . A[Ks, js]            (MFMA)
//   T hand-off within the XCD: the S workgroups of slice js run on one XCD
//          (workgroups are dealt to XCDs round-robin, which the host checks
//          at start-up); each publishes its partial through that XCD's L2
//          with an epoch flag, and every member sums the S partials in
//          order s = 0..S-1 (bitwise identical in every member).  Without a
//          verified XCD map the same exchange runs device-coherent.
//   GEMM2  Y_js[:, Ns] = T_js . B[js, Ns]               (T as bf16 hi + lo)
//   Y reduce-scatter across XCDs: partials stored device-coherent, every
//          value beside a copy of the launch's epoch in the same 16-byte
//          word; member js of n-slice s polls its 1/Jw share of the
//          n-slice until the Jw partials carry the epoch, sums them in
//          order and writes bf16 Y.
// No atomics and no floating-point reordering: results are bitwise
// reproducible.  The epoch of a launch is the handle's generation word
// (ctrl[0]) plus one, read by every workgroup at entry; workgroup 0 stores
// it back at its end.  Workgroup 0 finishes only after the Y partials of
// all rank slices of its n-slice, each of which followed the T flags of every
// K slice of that rank slice, so by then every workgroup of the launch has
// read the word.  No counter is reset between calls and no argument
// changes from one launch to the next, so a captured graph can replay the
// launch.
//
// Every row run is loaded from its exact first element (16-byte direct
// loads at any 2-byte offset), so a misaligned rank or width takes the same
// instructions as an aligned one: no code depends on the leading dimension
// modulo 8.  The buffer range check zeroes a dword that reaches past the
// matrix, so the workgroup whose slab holds the last element of A or of B
// writes it into LDS from a scalar load.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

namespace {

// Byte offset past the end of every buffer range used here: the load
// returns zeros (and writes them to LDS) without any branch.
constexpr uint32_t kOutOfRange = 0x7FFFFF00u;

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Weight and activation slabs are read once: non-temporal (streaming) loads,
// so that the XCD's L2 keeps the small T partials the group exchanges
// instead of the 4 MB per XCD of A and B passing through it.
__device__ __forceinline__ void lds_load16(rsrc_t r, void* lds_base_wave, uint32_t gbyte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_base_wave, 16, (int)gbyte_off, 0, 0, kSkipL1);
}

// Direct loads of `rows` runs of `cpr` 16-byte chunks into LDS slots
// [0, rows * cpr) of `lds` (run q at slot q * cpr).  Run q starts exactly at
// element e_first + q * ld; of each run only the chunks that hold its
// `ncols` elements are fetched, and runs q >= valid rows read as zero.  This wave issues load instructions first, first +
// step, ... (64 slots each).  The slot -> (run, chunk) map advances by a
// constant per instruction, so no division is done per load; element
// offsets fit 32 bits (matrices are below 2 GiB).
__device__ __forceinline__ void dma_runs(rsrc_t r, char* lds, uint32_t e_first, uint32_t ld, int rows, int valid,
                                         int cpr, int ncols, int first, int step, int lane) {
  const int ninst = (rows * cpr + 63) / 64;
  const int s0 = 64 * first + lane;
  int row = s0 / cpr, cc = s0 - row * cpr;
  const int adv = 64 * step;
  const int drow = adv / cpr, dcc = adv - drow * cpr;
  uint32_t e0 = e_first + (uint32_t)row * ld;
  const uint32_t dld = (uint32_t)drow * ld;
  for (int i = first; i < ninst; i += step) {
    const int need = (max(ncols, 0) + 7) >> 3;
    const bool ok = row < valid && cc < need;
    lds_load16(r, lds + i * 1024, ok ? (e0 + 8u * (uint32_t)cc) * 2u : kOutOfRange);
    row += drow;
    cc += dcc;
    e0 += dld;
    if (cc >= cpr) {
      cc -= cpr;
      row += 1;
      e0 += ld;
    }
  }
}

__device__ __forceinline__ u32x4_t lds_read16(const char* p) { return *reinterpret_cast<const u32x4_t*>(p); }
__device__ __forceinline__ void lds_write16(char* p, const u32x4_t& v) { *reinterpret_cast<u32x4_t*>(p) = v; }

// 8 rows held as chunk runs in LDS (row q at rows + q * pitch) -> 8 MFMA
// B-operands, in two steps so that the LDS reads of the next tile can be in
// flight while this one is transposed.  lane16 reads chunk c_off + lane16 of
// each run.  No masking here: rows past the matrix are zero in LDS, and
// output columns past the slice or the matrix are dropped by the callers.
struct TileRaw {
  u32x4_t lo[8];
};
__device__ __forceinline__ void tile_read(const char* rows, int pitch, int c_off, int lane16, TileRaw& t) {
#pragma unroll
  for (int q = 0; q < 8; ++q) t.lo[q] = lds_read16(rows + q * pitch + (c_off + lane16) * 16);
}
__device__ __forceinline__ void tile_ops(const TileRaw& t, u32x4_t op[8]) { transpose8x8(t.lo, op); }

struct ResCtx {
  const char* sA;
  const char* sB;
  const char* sX;
  int w, g, np;
  int kt_cnt, CB;
  int64_t kbase, j0, jend, K, r, N, nb0;
};

// GEMM1 partial over this wave's k-tiles t = w and w + 4 (a workgroup holds
// at most 8 k-tiles).  Both tiles are always computed: the LDS rows of tiles
// past kt_cnt are zero and their X operand is cleared, so they add exact
// zeros.  (Straight-line MFMA code keeps the accumulators in place; a
// conditional block around the MFMAs made the compiler shuffle them right
// behind each MFMA.)
__device__ __forceinline__ void gemm1_wave(const ResCtx& c, f32x4_t acc[8]) {
  const int pitch = kResCA * 16;
  TileRaw rt[2];
  u32x4_t xt[2];
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = c.w + 4 * h;
    tile_read(c.sA + (size_t)(t * kResKT + 8 * c.g) * pitch, pitch, 0, c.np, rt[h]);
    xt[h] = lds_read16(c.sX + c.np * (kResXK * 2) + (t * kResKT + 8 * c.g) * 2);
  }
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    const int t = c.w + 4 * h;
    u32x4_t op[8];
    tile_ops(rt[h], op);
    // X columns >= K (and tiles past kt_cnt) contribute zero
    const int64_t k0 = c.kbase + (int64_t)t * kResKT + 8 * c.g;
    const u32x4_t x = (t < c.kt_cnt && k0 < c.K) ? xt[h] : zerou4();
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[e] = mfma_16x16x32(x, op[e], acc[e]);
  }
}

// GEMM2 partials of this workgroup's two 128-column n-tiles for this wave's
// 32 rank rows (the second is computed even when the workgroup has one
// n-tile and is then never stored).
__device__ __forceinline__ void gemm2_wave(const ResCtx& c, const u32x4_t& thi, const u32x4_t& tlo, f32x4_t y0[8],
                                           f32x4_t y1[8]) {
  const char* rows = c.sB + (size_t)(32 * c.w + 8 * c.g) * (c.CB * 16);
  TileRaw b[2];
  tile_read(rows, c.CB * 16, 0, c.np, b[0]);
  tile_read(rows, c.CB * 16, 16, c.np, b[1]);
#pragma unroll
  for (int h = 0; h < 2; ++h) {
    u32x4_t op[8];
    tile_ops(b[h], op);
    f32x4_t* y = h == 0 ? y0 : y1;
#pragma unroll
    for (int e = 0; e < 8; ++e) {
      y[e] = mfma_16x16x32(thi, op[e], y[e]);
      y[e] = mfma_16x16x32(tlo, op[e], y[e]);
    }
  }
}

}  // namespace

// Optional phase timestamps (constant-rate device clock), compiled in only
// with -DLR_DECODE_TRACE.  They are held in scalar registers and stored at
// the end of the kernel, so that no trace store sits in the vector-memory
// counter that the phases wait on.
#ifdef LR_DECODE_TRACE
#define RES_TRACE_ENTRY()          \
  uint64_t trace_t_[16] = {};      \
  trace_t_[15] = res_trace_now()
#define RES_TRACE_ENTRY_STORE() do { } while (0)
#define RES_TRACE(i) trace_t_[i] = res_trace_now()
#define RES_TRACE_FLUSH()                                                                    \
  do {                                                                                       \
    if (a.trace && tid == 0)                                                                 \
      for (int i_ = 0; i_ < 16; ++i_) a.trace[blockIdx.x * kDecTracePoints + i_] = trace_t_[i_]; \
  } while (0)
__device__ __forceinline__ uint64_t res_trace_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : : "memory");
  return t;
}
#else
#define RES_TRACE_ENTRY() do { } while (0)
#define RES_TRACE_ENTRY_STORE() do { } while (0)
#define RES_TRACE(i) \
  do {               \
  } while (0)
#define RES_TRACE_FLUSH() do { } while (0)
#endif

__global__ __launch_bounds__(kResThreads) void lr_decode_res_kernel(const DecArgs a) {
  RES_TRACE_ENTRY();
  extern __shared__ __attribute__((aligned(16))) char smem[];

  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);  // wave-uniform: scalar branches
  const int l = tid & 63, np = l & 15, g = l >> 4;

  int pi = 0;
#pragma unroll
  for (int i = 1; i < kDecMaxProj; ++i)
    if (i < a.nproj && (int)blockIdx.x >= a.p[i].wg_begin) pi = i;
  const DecProj P = a.p[pi];
  const int local = (int)blockIdx.x - P.wg_begin;
  // Workgroup -> (rank slice, K/N slice).  With the XCD map, the S members of
  // a rank slice share local % 8 and so run on one XCD.
  int js, s;
  if (P.xcd_local) {
    const int x = local & 7, slot = local >> 3;
    js = x * (P.Jw >> 3) + slot / P.S;  // each XCD holds adjacent rank slices (shared A lines)
    s = slot - (slot / P.S) * P.S;
  } else {
    js = local / P.S;
    s = local - js * P.S;
  }
  const int M = a.M, K = a.K, r = P.r, N = P.N;
  const int JS = P.js_w;
  const int ntps = P.ntps;
  const int CB = kResNT / 8 * ntps + 1;  // chunks per B row run
  // the generation word is requested here and first used after A has landed
  const uint32_t gen_v = ld_agent_u32(P.ctrl);

  const rsrc_t rA = make_rsrc(P.A, (int64_t)K * r * 2);
  const rsrc_t rB = make_rsrc(P.B, (int64_t)r * N * 2);
  const rsrc_t rX = make_rsrc(a.X, (int64_t)M * K * 2);
  const rsrc_t rW = make_rsrc(P.ws, P.ws_bytes);

  char* const sX = smem;               // [16][kResXK] bf16, row pitch kResXK*2
  char* const sA = smem + kResXBytes;  // [ktps*32][kResCA] chunks
  char* const sB = sA + kResABytes;    // [128][CB] chunks
  float* const red = reinterpret_cast<float*>(sA);                 // after GEMM1: [4][16][128]
  float* const Ts = reinterpret_cast<float*>(sA + kResRedBytes);  // [16][136]

  const int64_t j0 = (int64_t)js * JS;
  const int64_t jend = min64(r, j0 + JS);
  const int nk = (K + kResKT - 1) / kResKT;
  const int kt_beg = s * P.ktps;
  const int kt_cnt = max(0, min(nk, kt_beg + P.ktps) - kt_beg);
  const int64_t kbase = (int64_t)kt_beg * kResKT;
  const int nn = (N + kResNT - 1) / kResNT;
  const int nt_beg = s * ntps;
  const int nt_cnt = max(0, min(nn, nt_beg + ntps) - nt_beg);
  const int64_t nb0 = (int64_t)nt_beg * kResNT;

  RES_TRACE(0);
  RES_TRACE_ENTRY_STORE();

  // LDS rows of the B slab past the slice are never loaded.  GEMM2 multiplies
  // them by T columns that are exactly zero, so they are cleared here: bits
  // left by an earlier kernel could be NaN or Inf.  (The B loads below write
  // only zeros there, so the order of the two does not matter.)
  {
    const int r0 = (int)(jend - j0);
    const int nz = (kResJS - r0) * CB;
    for (int i = tid; i < nz; i += kResThreads) lds_write16(sB + ((size_t)r0 * CB + i) * 16, zerou4());
    // likewise the A rows of k-tiles past kt_cnt (GEMM1 always runs 8 tiles)
    const int az = (kResMaxKt - kt_cnt) * kResKT * kResCA;
    for (int i = tid; i < az; i += kResThreads)
      lds_write16(sA + ((size_t)kt_cnt * kResKT * kResCA + i) * 16, zerou4());
  }

  // ------------------------------------------- X and A straight to LDS --
  if (w < 2) {
    // X: 16 rows x kResXK columns starting at kbase (rows >= M read as zero)
    dma_runs(rX, sX, (uint32_t)kbase, (uint32_t)K, 16, M, kResXK / 8, kResXK, w, 2, l);
    // A: kt_cnt*32 rows, each a run of kResCA chunks starting at the chunk
    // that holds column j0 of the row; rows >= K read as zero
    dma_runs(rA, sA, (uint32_t)(kbase * r + j0), (uint32_t)r, kt_cnt * kResKT, (int)min64(kt_cnt * kResKT, K - kbase),
             kResCA, (int)(jend - j0), w, 2, l);
  }
  wait_vmem_all();
  barrier_lds();  // X and A are in LDS
  // A's last element (K - 1, r - 1), if this workgroup's slab holds it (see the top)
  if (jend == r && kt_cnt > 0 && kbase + (int64_t)kt_cnt * kResKT >= K) {
    if (tid == 0)
      *reinterpret_cast<uint16_t*>(sA + (size_t)(K - 1 - kbase) * kResCA * 16 + (r - 1 - j0) * 2) =
          (uint16_t)scalar_elem(P.A, (int64_t)K * r - 1);
    barrier_lds();
  }
  const uint32_t gen = __builtin_amdgcn_readfirstlane(gen_v);
  const uint32_t epoch = gen + 1u == 0u ? 1u : gen + 1u;  // 0 is the value of a fresh flag
  RES_TRACE(1);
  ResCtx ctx;
  ctx.sA = sA;
  ctx.sB = sB;
  ctx.sX = sX;
  ctx.w = w;
  ctx.g = g;
  ctx.np = np;
  ctx.kt_cnt = kt_cnt;
  ctx.CB = CB;
  ctx.kbase = kbase;
  ctx.j0 = j0;
  ctx.jend = jend;
  ctx.K = K;
  ctx.r = r;
  ctx.N = N;
  ctx.nb0 = nb0;

  // ---------------------------------------------------------- GEMM1 ------
  f32x4_t acc[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) acc[e] = zero4();
  gemm1_wave(ctx, acc);
  RES_TRACE(2);
  barrier_lds();  // every wave is done reading A: the A region is free
#pragma unroll
  for (int e = 0; e < 8; ++e)
#pragma unroll
    for (int t = 0; t < 4; ++t) red[(w * 16 + 4 * g + t) * 128 + 8 * np + e] = acc[e][t];
  barrier_lds();

  // ------------------------------------------- publish the T partial -----
  // slice layout: [M][128] fp32 (columns >= JS unused)
  const int v4row = JS / 4;
  const int nvecT = M * v4row;
  const uint32_t slice_bytes = (uint32_t)(M * 128 * 4);
  const uint32_t grp_base = P.off_tpart + (uint32_t)(js * P.S) * slice_bytes;
  if (w < 2) {
    for (int vi = tid; vi < nvecT; vi += 128) {
      const int m = vi / v4row, c = (vi - m * v4row) * 4;
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = m * 128 + c + i;
        const float t = ((red[o] + red[16 * 128 + o]) + red[32 * 128 + o]) + red[48 * 128 + o];
        v[i] = c + i < jend - j0 ? t : 0.f;  // columns past the slice (or r) are exactly zero
      }
      const uint32_t off = grp_base + (uint32_t)s * slice_bytes + (uint32_t)(m * 128 + c) * 4u;
      if (P.xcd_local)
        buf_store16(rW, off, v);
      else
        buf_store16_coherent(rW, off, v);
    }
    wait_vmem_all();  // the partial is visible before the flag
  }
  barrier_lds();
  const uint32_t tflag_grp = P.off_tflag + (uint32_t)(js * P.S) * 4u;
  if (tid == 0) {
    if (P.xcd_local)
      buf_store_u32(rW, tflag_grp + (uint32_t)s * 4u, epoch);
    else
      buf_store_u32_coherent(rW, tflag_grp + (uint32_t)s * 4u, epoch);
  }
  RES_TRACE(3);
  // B is requested only now: A had the memory system to itself, and the T
  // partial stores above did not queue behind B's requests.  B is needed
  // only at GEMM2 and streams in during the T hand-off.
  if (w >= 2) {
    // B: the slice's rows, each a run of CB chunks starting at the chunk
    // that holds column nb0 of the row (LDS rows past the slice are cleared
    // above)
    dma_runs(rB, sB, (uint32_t)(j0 * N + nb0), (uint32_t)N, (int)(jend - j0), (int)(jend - j0), CB,
             (int)min64((int64_t)nt_cnt * kResNT, N - nb0), w - 2, 2, l);
  }


  // ------------------------------------ T hand-off: all S partials -------
  if (w == 0) {
    uint32_t spins = 0;
    while (true) {
      bool ok = true;
      for (int i = l; i < P.S; i += 64) {
        const uint32_t f = P.xcd_local ? buf_load_u32_l2(rW, tflag_grp + (uint32_t)i * 4u)
                                       : buf_load_u32_coherent(rW, tflag_grp + (uint32_t)i * 4u);
        ok = ok && (f == (epoch ^ P.stall_xor));
      }
      if (__all(ok)) break;
      if (++spins > P.spin_limit) {
        if (l == 0) raise_stall(P.ctrl, P.err);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
  }
  barrier_lds();
  RES_TRACE(4);
  // thread -> float4 element of the slice (M x JS valid floats); all S
  // partials of it in flight, summed in order s = 0..S-1.  Ts is cleared
  // first: rows >= M and columns >= JS are zero for GEMM2.
  for (int idx = tid; idx < 16 * 136; idx += kResThreads) Ts[idx] = 0.f;
  barrier_lds();
  {
    const int v4row = JS / 4;
    for (int vi = tid; vi < M * v4row; vi += kResThreads) {
      const int m = vi / v4row, c = (vi - m * v4row) * 4;
      const uint32_t voff = (uint32_t)(m * 128 + c) * 4u;
      f32x4_t sum = zero4();
      for (int p0 = 0; p0 < P.S; p0 += 16) {
        const int np0 = min(16, P.S - p0);
        f32x4_t t[16];
#pragma unroll
        for (int u = 0; u < 16; ++u) {
          const uint32_t off = grp_base + (uint32_t)(p0 + min(u, np0 - 1)) * slice_bytes + voff;
          if (u < np0) t[u] = P.xcd_local ? buf_load16_fresh(rW, off) : buf_load16_coherent(rW, off);
        }
#pragma unroll
        for (int u = 0; u < 16; ++u)
          if (u < np0) sum += t[u];
      }
#pragma unroll
      for (int i = 0; i < 4; ++i)
        if (c + i < JS) Ts[m * 136 + c + i] = sum[i];
    }
  }
  RES_TRACE(9);
  wait_vmem_all();  // B (loaded by waves 2-3) is in LDS
  barrier_lds();
  // B's last element (r - 1, N - 1), if this workgroup's slab holds it
  if (jend == r && nt_cnt > 0 && nb0 + (int64_t)nt_cnt * kResNT >= N) {
    if (tid == 0)
      *reinterpret_cast<uint16_t*>(sB + (size_t)(r - 1 - j0) * CB * 16 + (N - 1 - nb0) * 2) =
          (uint16_t)scalar_elem(P.B, (int64_t)r * N - 1);
    barrier_lds();
  }
  RES_TRACE(5);

  // bf16 hi/lo split of this wave's 32 rank rows: lane (i = np, g) holds
  // T[i][32w + 8g + q], q = 0..7.
  u32x4_t thi, tlo;
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    const float t0v = Ts[np * 136 + 32 * w + 8 * g + 2 * p];
    const float t1v = Ts[np * 136 + 32 * w + 8 * g + 2 * p + 1];
    const uint32_t h0 = f32_to_bf16_rne(t0v), h1 = f32_to_bf16_rne(t1v);
    thi[p] = h0 | (h1 << 16);
    tlo[p] = pack_bf16x2(t0v - __uint_as_float(h0 << 16), t1v - __uint_as_float(h1 << 16));
  }

  // ---------------------------------------------------------- GEMM2 ------
  // Y partial layout per (s, js): [nt][M][128] fp32 = ntps*M*32 float4, each
  // stored as two epoch-tagged exchange words (lr_device.h), polled by the
  // reduce-scatter below: no flag and no wait for the stores to complete.
  const int vmax = ntps * M * 32;
  const uint32_t ypart_wg = P.off_ypart + (uint32_t)(s * P.Jw + js) * (uint32_t)vmax * 32u;
  const float tagf = __uint_as_float(epoch);
  f32x4_t y0[8], y1[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    y0[e] = zero4();
    y1[e] = zero4();
  }
  gemm2_wave(ctx, thi, tlo, y0, y1);
  RES_TRACE(10);
  for (int ntl = 0; ntl < nt_cnt; ++ntl) {
    barrier_lds();  // previous tile's red reads (and the Ts reads) are done
#pragma unroll
    for (int e = 0; e < 8; ++e)
#pragma unroll
      for (int t = 0; t < 4; ++t) red[(w * 16 + 4 * g + t) * 128 + 8 * np + e] = ntl == 0 ? y0[e][t] : y1[e][t];
    barrier_lds();
    for (int vi = tid; vi < M * 32; vi += kResThreads) {
      const int m = vi >> 5, c = (vi & 31) * 4;
      f32x4_t v;
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int o = m * 128 + c + i;
        v[i] = ((red[o] + red[16 * 128 + o]) + red[32 * 128 + o]) + red[48 * 128 + o];
      }
      const uint32_t off = ypart_wg + (uint32_t)(ntl * M * 32 + vi) * 32u;
      xstore_coherent(rW, off, v[0], v[1], tagf);
      xstore_coherent(rW, off + 16u, v[2], v[3], tagf);
    }
  }
  RES_TRACE(6);

  // -------------------------------- Y reduce-scatter over the Jw slices --
  if (nt_cnt > 0) {
    RES_TRACE(11);
    // my share of the n-slice: value pairs [q_lo, q_hi) of nt_cnt*M*64 (pair
    // q is the tagged word at byte 16 q of a partial); each thread polls the
    // Jw partials of a pair until every tag holds this launch's epoch and
    // sums them in order.
    const int qtot = nt_cnt * M * 64;
    const int share = (qtot + P.Jw - 1) / P.Jw;
    const int q_lo = js * share;
    const int q_hi = min(qtot, q_lo + share);
    const uint32_t grp_y = P.off_ypart + (uint32_t)(s * P.Jw) * (uint32_t)vmax * 32u;
    for (int q = q_lo + tid; q < q_hi; q += kResThreads) {
      float s0, s1;
      xpoll_sum(rW, grp_y, (uint32_t)vmax * 32u, P.Jw, (uint32_t)q * 16u, epoch, P.spin_limit, P.ctrl, P.err, s0, s1);
      const int vi = q >> 1;
      const int ntl = vi / (M * 32);
      const int rem = vi - ntl * M * 32;
      const int m = rem >> 5, c = (rem & 31) * 4 + 2 * (q & 1);
      const int64_t n0 = nb0 + (int64_t)ntl * kResNT + c;
      if (n0 < N) P.Y[(int64_t)m * N + n0] = (uint16_t)f32_to_bf16_rne(s0);
      if (n0 + 1 < N) P.Y[(int64_t)m * N + n0 + 1] = (uint16_t)f32_to_bf16_rne(s1);
    }
    RES_TRACE(7);
  }
  RES_TRACE(8);
  if (local == 0 && tid == 0) st_agent_u32(P.ctrl, epoch);  // the next launch's generation
  RES_TRACE_FLUSH();
}

hipError_t launch_decode_res(const DecArgs& args, int grid, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  static std::atomic<uint64_t> occ{0};
  hipError_t e = ensure_dynamic_lds((const void*)lr_decode_res_kernel, kResLdsBytes, attr_done);
  if (e == hipSuccess) e = check_coresident((const void*)lr_decode_res_kernel, kResThreads, kResLdsBytes, grid, occ);
  if (e != hipSuccess || args.check_only) return e;
  hipLaunchKernelGGL(lr_decode_res_kernel, dim3(grid), dim3(kResThreads), kResLdsBytes, stream, args);
  return hipGetLastError();
}

bool decode_res_available() {
  int dev = 0, lds = 0;
  if (hipGetDevice(&dev) != hipSuccess) return false;
  if (hipDeviceGetAttribute(&lds, hipDeviceAttributeMaxSharedMemoryPerBlock, dev) != hipSuccess) return false;
  return lds >= kResLdsBytes;
}

// Records HW_REG_XCC_ID of each workgroup of a grid.
__global__ void xcc_map_kernel(uint32_t* out) {
  if (threadIdx.x == 0) out[blockIdx.x] = xcc_id();
}

bool xcd_round_robin(int grid) {
  uint32_t* d = nullptr;
  if (hipMalloc(&d, (size_t)grid * 4) != hipSuccess) return false;
  bool ok = false;
  hipLaunchKernelGGL(xcc_map_kernel, dim3(grid), dim3(64), 0, 0, d);
  uint32_t* h = new uint32_t[grid];
  if (hipGetLastError() == hipSuccess && hipMemcpy(h, d, (size_t)grid * 4, hipMemcpyDeviceToHost) == hipSuccess) {
    ok = true;
    for (int i = 0; i < grid; ++i) ok = ok && (h[i] == (uint32_t)(i & 7));
  }
  delete[] h;
  (void)hipFree(d);
  return ok;
}

}  // namespace lrk
