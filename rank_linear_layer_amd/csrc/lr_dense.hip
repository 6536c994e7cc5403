// Dense fallback: Y = X . W with W = A . B formed once when the handle is
// created, for shapes where the factorization saves (almost) no weight bytes
// ("LowRankArena: What Happens When You Force SVD Compression Papers to Play
// by the Same Rules", Q3: The FLOP-savings-to-latency gap, on a method that
// runs a layer as one dense GEMM when its retained rank saves no memory
// bandwidth).  The k/v projections of the Llama-3-8B-shaped layer at
// r = 817 hold 99.7% of the dense bytes.
//
// W itself is computed by the prefill GEMM (P = A, Q = B).  This file holds
// the two pieces that are specific to the dense path:
//
//  * lr_dense_swizzle_kernel: W (row-major K x N) -> Wsw, the decode layout.
//    Column group g (16 columns) and k-step s (32 rows) form one 1 KB block,
//    blocks of a group stored consecutively; inside a block lane l holds the
//    16 bytes W[32 s + 8 (l / 16) + 0..7][16 g + l % 16], which is exactly
//    the B operand of a 16x16x32 bf16 MFMA.  Rows >= K and columns >= N are
//    zero.
//
//  * lr_dense_decode_kernel (M <= 16, HBM-bound): the column groups of every
//    output sharing X in the launch, each cut into `splits` slices of K
//    where the host finds the groups too few and too deep (a K = 14336
//    layer: 64 groups of 448 k-steps, 14.3 us as one slice, 10.8 us as four
//    on MI355X; the k/v shape, 64 groups of 128 k-steps, takes the same
//    7.3 us as one or two slices and gets slower with more: a launch of
//    8 MB is bound by latency, not by how many compute units stream).
//    Workgroup (slice, group) reads its
//    part of the group's K x 16 slab of Wsw as whole 1 KB blocks (each wave
//    instruction is one contiguous kilobyte) and multiplies it by X; the
//    eight waves split the slice and their 16 x 16 partials are summed in
//    LDS in wave order.  With one slice the tile is written as bf16.
//    Otherwise it is stored as an fp32 partial (device-coherent), and the
//    workgroup counts itself in on the group's counter; the last to arrive
//    adds the group's partials in slice order 0, 1, ... (the same order
//    whichever workgroup is last, so results are reproducible bit for bit),
//    writes bf16 and resets the counter.  No workgroup ever waits for
//    another, so the launch completes whatever runs concurrently.
#include "lr_device.h"
#include "lr_kernels.h"

namespace lrk {

namespace {

constexpr int kDnThreads = 512;  // 8 waves
constexpr int kDnWaves = kDnThreads / 64;
constexpr int kDnChunk = 16;     // k-steps whose operands are in flight at once per wave

}  // namespace

__global__ __launch_bounds__(256) void lr_dense_swizzle_kernel(const uint16_t* W, uint16_t* Wsw, int64_t K, int64_t N,
                                                               int64_t nk, int64_t nblocks) {
  const int64_t t = (int64_t)blockIdx.x * 256 + threadIdx.x;  // (block, lane)
  const int64_t blk = t >> 6;
  if (blk >= nblocks) return;
  const int l = (int)(t & 63);
  const int64_t g = blk / nk, s = blk - g * nk;
  const int64_t col = 16 * g + (l & 15);
  const int64_t row0 = 32 * s + 8 * (l >> 4);
  uint32_t e[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) {
    const int64_t row = row0 + j;
    e[j] = (row < K && col < N) ? (uint32_t)W[row * N + col] : 0u;
  }
  u32x4_t v;
#pragma unroll
  for (int p = 0; p < 4; ++p) v[p] = e[2 * p] | (e[2 * p + 1] << 16);
  *reinterpret_cast<u32x4_t*>(Wsw + t * 8) = v;
}

// XAL: K is a multiple of 8 (X rows are 16-byte aligned).  A compile-time
// choice: a branch around the loads would make the compiler wait for every
// load in flight where the branches join.
template <bool XAL>
__global__ __launch_bounds__(kDnThreads) void lr_dense_decode_kernel(const DenseArgs a) {
  __shared__ __align__(16) float red[kDnWaves][256];
  __shared__ uint32_t sh_old;
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  // (slice, column group) of this workgroup: slice-major, then the
  // outputs' groups in order
  const int split = (int)(blockIdx.x / a.ng);
  int64_t g = (int64_t)blockIdx.x - (int64_t)split * a.ng;
  int oi = 0;
#pragma unroll
  for (int i = 0; i < kDenseMaxOut - 1; ++i) {
    const int64_t ng = (a.o[oi].N + 15) / 16;
    if (oi + 1 < a.nout && g >= ng) {
      g -= ng;
      ++oi;
    }
  }
  const DenseOut& o = a.o[oi];
  const int64_t nk = a.nk;
  // this workgroup's k-steps [k0, k1), and this wave's share [s0, s1)
  const int64_t k0 = nk * split / a.splits, k1 = nk * (split + 1) / a.splits;
  const int64_t per = (k1 - k0 + kDnWaves - 1) / kDnWaves;
  const int64_t s0 = min64(k1, k0 + (int64_t)w * per), s1 = min64(k1, s0 + per);

  const rsrc_t rW = make_rsrc(o.Wsw + g * nk * 512, nk * 1024);
  const rsrc_t rX = make_rsrc(a.X, (int64_t)a.M * a.K * 2);
  // A operand of lane l: row m = l % 16 of X (rows >= M read as zero),
  // columns 32 s + 8 (l / 16) .. + 7.  With K a multiple of 8 that is one
  // aligned 16-byte load; otherwise the two aligned chunks around it are
  // loaded and the lane realigns them by its row's offset.
  const int m = l & 15;
  const int64_t xrow = (int64_t)m * a.K;
  const int d = (int)(xrow & 7);

  f32x4_t acc = zero4();
  for (int64_t c0 = s0; c0 < s1; c0 += kDnChunk) {
    u32x4_t wv[kDnChunk], xl[kDnChunk], xh[kDnChunk];
#pragma unroll
    for (int i = 0; i < kDnChunk; ++i) {
      // steps past s1 read block offsets past this group's range: zeros
      const int64_t s = c0 + i;
      wv[i] = buf_load16(rW, (uint32_t)(s < s1 ? (s * 1024 + l * 16) : nk * 1024));
      const int64_t e = xrow + 32 * s + 8 * (l >> 4);
      if (XAL) {
        xl[i] = buf_load16(rX, (uint32_t)(e * 2));
      } else {
        xl[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16));
        xh[i] = buf_load16(rX, (uint32_t)((e >> 3) * 16 + 16));
      }
    }
#pragma unroll
    for (int i = 0; i < kDnChunk; ++i) {
      // columns >= K (the next row's elements, or bytes past X) and rows
      // >= M are cleared: rows of W past K are zero, but 0 * NaN is not
      const u32x4_t x = mask_cols(XAL ? xl[i] : realign_lane(xl[i], xh[i], d), 32 * (c0 + i) + 8 * (l >> 4), a.K);
      acc = mfma_16x16x32(m < a.M ? x : zerou4(), wv[i], acc);
    }
  }
  // acc lane l, register t: row 4 (l / 16) + t, column l % 16
#pragma unroll
  for (int t = 0; t < 4; ++t) red[w][(4 * (l >> 4) + t) * 16 + (l & 15)] = acc[t];
  __syncthreads();
  // thread t < 64: elements 4t .. 4t + 3 of the 16 x 16 tile (row t / 4)
  const int row = tid >> 2, col = 4 * (tid & 3);
  auto store_y = [&](const f32x4_t& v) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int64_t n = 16 * g + col + i;
      if (row < a.M && n < o.N) o.Y[(int64_t)row * o.N + n] = (uint16_t)f32_to_bf16_rne(v[i]);
    }
  };
  f32x4_t v = zero4();
  if (tid < 64) {
#pragma unroll
    for (int i = 0; i < kDnWaves; ++i) {
      const f32x4_t p = *reinterpret_cast<const f32x4_t*>(&red[i][4 * tid]);
#pragma unroll
      for (int e = 0; e < 4; ++e) v[e] += p[e];
    }
  }
  if (a.splits == 1) {
    if (tid < 64) store_y(v);
    return;
  }
  const int64_t ngo = (o.N + 15) / 16;
  const rsrc_t rP = make_rsrc(o.part, (int64_t)a.splits * ngo * 1024);
  if (tid < 64) buf_store16_coherent(rP, (uint32_t)(((int64_t)split * ngo + g) * 1024 + tid * 16), v);
  wait_vmem_all();
  barrier_lds();
  if (tid == 0) sh_old = add_agent_u32(o.cnt + g, 1u);
  barrier_lds();
  if (sh_old != (uint32_t)(a.splits - 1)) return;
  // the last of the group's workgroups: every partial is stored
  if (tid == 0) st_agent_u32(o.cnt + g, 0u);
  if (tid < 64) {
    f32x4_t s = zero4();
    for (int q = 0; q < a.splits; ++q) {
      const f32x4_t p = buf_load16_coherent(rP, (uint32_t)(((int64_t)q * ngo + g) * 1024 + tid * 16));
#pragma unroll
      for (int e = 0; e < 4; ++e) s[e] += p[e];
    }
    store_y(s);
  }
}

hipError_t launch_dense_swizzle(const uint16_t* W, uint16_t* Wsw, int64_t K, int64_t N, hipStream_t stream) {
  const int64_t nk = (K + 31) / 32, ng = (N + 15) / 16;
  const int64_t nblocks = nk * ng;
  const int64_t threads = nblocks * 64;
  const int64_t grid = (threads + 255) / 256;
  if (grid <= 0) return hipSuccess;
  if (grid > 0x7FFFFFFF) return hipErrorInvalidValue;
  hipLaunchKernelGGL(lr_dense_swizzle_kernel, dim3((unsigned)grid), dim3(256), 0, stream, W, Wsw, K, N, nk, nblocks);
  return hipGetLastError();
}

hipError_t launch_dense_decode(const DenseArgs& args, hipStream_t stream) {
  if (args.M <= 0) return hipSuccess;
  if (args.nout < 1 || args.nout > kDenseMaxOut || args.M > 16 || args.nk != (args.K + 31) / 32 ||
      args.splits < 1 || args.splits > kDenseMaxSplits || args.splits > args.nk)
    return hipErrorInvalidValue;
  int64_t ng = 0;
  for (int i = 0; i < args.nout; ++i) {
    if (args.o[i].N < 1) return hipErrorInvalidValue;
    if (args.splits > 1 && (!args.o[i].part || !args.o[i].cnt)) return hipErrorInvalidValue;
    ng += (args.o[i].N + 15) / 16;
  }
  if (ng != args.ng || ng * args.splits > 0x7FFFFFFF) return hipErrorInvalidValue;
  const dim3 grid((unsigned)(ng * args.splits));
  if ((args.K & 7) == 0)
    hipLaunchKernelGGL(lr_dense_decode_kernel<true>, grid, dim3(kDnThreads), 0, stream, args);
  else
    hipLaunchKernelGGL(lr_dense_decode_kernel<false>, grid, dim3(kDnThreads), 0, stream, args);
  return hipGetLastError();
}

}  // namespace lrk
