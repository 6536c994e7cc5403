// Prefill kernels (M > 16): MFMA GEMMs with on-chip rank padding.
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
// their public shapes.  The N edge is masked in the epilogue.  No kernel
// variant depends on r mod 8 or N mod 8.
//
// One launch of lr_prefill_gemm_kernel computes one phase; for a gate/up pair
// phase 1 covers both factor pairs in the same launch (column tiles of both
// outputs share the row tiles of X).
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

struct PreRaw {
  u32x4_t c[8];
};

__device__ __forceinline__ void pre_load_raw(PreRaw& t, rsrc_t rQ, int64_t kb, int64_t ldq, int64_t colbase,
                                             int lane16, int g) {
#pragma unroll
  for (int q = 0; q < 8; ++q) t.c[q] = load_row_raw(rQ, kb + 8 * g + q, ldq, colbase, lane16);
}

// Rows past the end of Q already read as zero (buffer range), so every row
// of the tile is kept.
__device__ __forceinline__ void pre_operands(const PreRaw& t, u32x4_t op[8], int64_t ldq, int64_t colbase,
                                             int lane16) {
  u32x4_t seg[8];
#pragma unroll
  for (int q = 0; q < 8; ++q) {
    const int d = (int)(((int64_t)q * ldq + colbase) & 7);
    seg[q] = realign_segment(t.c[q], d, colbase + 8 * lane16, ldq, true);
  }
  transpose8x8(seg, op);
}

__global__ __launch_bounds__(kPreThreads) void lr_prefill_gemm_kernel(const PreArgs a) {
  const int tid = threadIdx.x;
  const int w = tid >> 6, l = tid & 63, np = l & 15, g = l >> 4;
  const int wm = w >> 1, wn = w & 1;

  int bi = 0;
  int ct = blockIdx.x;
  if (a.nout > 1 && ct >= a.o[0].col_tiles) {
    bi = 1;
    ct -= a.o[0].col_tiles;
  }
  const PreOut O = a.o[bi];
  const int64_t mb = (int64_t)blockIdx.y * kPreBM + 64 * wm;
  const int64_t colbase = (int64_t)ct * kPreBN + 120 * wn;
  const rsrc_t rQ = make_rsrc(O.Q, O.qrows * O.ldq * 2);
  const rsrc_t rP = make_rsrc(O.P, a.rows * O.ldp * 2);
  const bool pal = (O.ldp & 7) == 0;

  f32x4_t acc[4][8];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int e = 0; e < 8; ++e) acc[i][e] = zero4();

  const int nks = (int)((O.kd + kPreKT - 1) / kPreKT);
  PreRaw r0, r1;
  u32x4_t x0[4], x1[4];
  auto load_step = [&](PreRaw& rr, u32x4_t* xx, int ks) {
    const int64_t kb = (int64_t)ks * kPreKT;
    pre_load_raw(rr, rQ, kb, O.ldq, colbase, np, g);
#pragma unroll
    for (int i = 0; i < 4; ++i) xx[i] = load_kvec(rP, mb + 16 * i + np, O.ldp, kb + 8 * g, O.kd, pal);
  };
  auto compute_step = [&](const PreRaw& rr, const u32x4_t* xx, int ks) {
    u32x4_t op[8];
    pre_operands(rr, op, O.ldq, colbase, np);
    const int64_t k0 = (int64_t)ks * kPreKT + 8 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const u32x4_t xm = kvec_mask(xx[i], k0, O.kd);
#pragma unroll
      for (int e = 0; e < 8; ++e) acc[i][e] = mfma_16x16x32(xm, op[e], acc[i][e]);
    }
  };

  if (nks > 0) load_step(r0, x0, 0);
  for (int ks = 0; ks < nks; ks += 2) {
    if (ks + 1 < nks) load_step(r1, x1, ks + 1);
    compute_step(r0, x0, ks);
    if (ks + 1 >= nks) break;
    if (ks + 2 < nks) load_step(r0, x0, ks + 2);
    compute_step(r1, x1, ks + 1);
  }

  // Epilogue: lane (np, g) of MFMA (i, e) holds rows mb + 16i + 4g + t,
  // column colbase + 8np + e.  Lane 15 carries no output column.
  if (np == 15) return;
  const int64_t col0 = colbase + 8 * np;
  if (col0 >= O.out_cols) return;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
#pragma unroll
    for (int t = 0; t < 4; ++t) {
      const int64_t row = mb + 16 * i + 4 * g + t;
      if (row >= a.rows) continue;
      u32x4_t v;
      v[0] = pack_bf16x2(acc[i][0][t], acc[i][1][t]);
      v[1] = pack_bf16x2(acc[i][2][t], acc[i][3][t]);
      v[2] = pack_bf16x2(acc[i][4][t], acc[i][5][t]);
      v[3] = pack_bf16x2(acc[i][6][t], acc[i][7][t]);
      uint16_t* dst = O.C + row * O.ldc + col0;
      if (col0 + 8 <= O.out_cols && ((row * O.ldc + col0) & 7) == 0) {
        *reinterpret_cast<u32x4_t*>(dst) = v;
      } else {
#pragma unroll
        for (int e = 0; e < 8; ++e) {
          if (col0 + e < O.out_cols) dst[e] = (uint16_t)(v[e >> 1] >> (16 * (e & 1)));
        }
      }
    }
  }
}

hipError_t launch_prefill_gemm(const PreArgs& args, hipStream_t stream) {
  int col_tiles = args.o[0].col_tiles + (args.nout > 1 ? args.o[1].col_tiles : 0);
  hipLaunchKernelGGL(lr_prefill_gemm_kernel, dim3(col_tiles, args.row_tiles), dim3(kPreThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace lrk
