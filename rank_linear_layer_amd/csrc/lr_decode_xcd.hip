// XCD-sliced fused decode kernel (M <= 16): Y = (X . A) . B in one launch,
// reading A [K x r] and B [r x N] in place, row-major, for any r and N.
//
// Decode reads every factor byte once and is bound by HBM ("LowRankArena
// ...", "Why theoretical FLOPs saved does not equal faster inference").  On
// this GPU a compute unit streams only a 1/256 share of the HBM rate, so the
// launch gives every compute unit (one workgroup each) an equal share of A
// AND of B, and keeps the hand-off of T = X . A inside each XCD:
//
//  * XCD x owns rank rows [x r / 8, (x + 1) r / 8) of the projection.  Its
//    pn workgroups split that range into rs sub-ranges and K into ks slabs
//    (ks rs = pn): workgroup (sub-range, slab) computes the fp32 partial T
//    of its sub-range over its slab (GEMM1), publishes it through the XCD's
//    L2 and, once every partial of the XCD is in, sums the ks partials of
//    each sub-range in slab order, so each workgroup holds T for the whole
//    rank range of its XCD.  T never leaves the XCD.
//  * Workgroup i of the XCD owns columns [i N / pn, (i + 1) N / pn) and
//    computes the partial Y = T[:, range] . B[range, columns] (GEMM2).  The
//    eight XCDs' partials of a column slab are then summed across XCDs in
//    XCD order (reduce-scatter: the slab's workgroup on XCD x sums and
//    stores the x-th eighth of its columns).
//
// Per workgroup, waves 0-3 (the A team) stream their k-steps of the A piece
// and do GEMM1 and the T exchange; waves 4-7 (the B team) request their
// columns of the B piece at entry, so that B streams in while T is formed,
// and do GEMM2.  Each wave consumes only what it loaded itself, so the
// in-order vector-memory counter of one wave never couples the two phases.
// Every factor load is a 16-byte direct-to-LDS load at the element's own
// address (rows of any alignment; the hardware splits unaligned accesses),
// and the MFMA operands are read with the transposing LDS read, so the
// rank is padded to the MFMA K-step and the N edge is masked on chip, with
// no copy of A or B anywhere.
//
// Reading unaligned 16-byte pieces through a buffer range zeroes every dword
// that reaches past the range, so the last element of a matrix can be lost
// when it is the low half of such a dword; the one wave whose piece holds it
// fetches it separately (2-byte load at entry) and patches it in.
//
// Exchanges are stamped with an epoch: the projection's generation word
// ctrl[0] plus one, read by every workgroup at entry.  Every workgroup counts
// itself out in ctrl[1] when done; the last one resets the count and stores
// the epoch as the next generation, so no host-side clearing is needed and a
// captured graph can replay the launch.  The launch assumes all of its
// workgroups are resident at once (one per compute unit; the launcher refuses
// a grid that does not fit), and each wait gives up after spin_limit polls,
// raising ctrl[2] and the host-visible error word instead of hanging.
#include "lr_device.h"
#include "lr_kernels.h"
#include "lr_ldsops.h"

namespace lrk {

namespace {

constexpr int kXThreads = 512;
constexpr uint32_t kXOut = 0x7FFFFF00u;  // past every buffer range: loads read zero
constexpr int kXcdMaxInst = 17;           // DMA instructions per k-step of a padded tile (32 x 33 chunks)

// Optional phase timestamps (constant-rate device clock), compiled in only
// with -DLR_DECODE_TRACE: waves 0 and 4 each keep 16 in registers and store
// them when the kernel ends (trace[(wg * 2 + team) * 16 + i]).
#ifdef LR_DECODE_TRACE
#define XT(i) tr[i] = xt_now()
__device__ __forceinline__ uint64_t xt_now() {
  uint64_t t;
  asm volatile("s_memrealtime %0\n\ts_waitcnt lgkmcnt(0)" : "=s"(t) : : "memory");
  return t;
}
#else
#define XT(i) \
  do {        \
  } while (0)
#endif

__device__ __forceinline__ void store_u16(rsrc_t r, uint32_t byte_off, uint32_t v) {
  __builtin_amdgcn_raw_buffer_store_b16((uint16_t)v, r, (int)byte_off, 0, 0);
}
template <int AUX>
__device__ __forceinline__ void store_f32(rsrc_t r, uint32_t byte_off, float v) {
  __builtin_amdgcn_raw_buffer_store_b32(__float_as_uint(v), r, (int)byte_off, 0, AUX);
}
template <int AUX>
__device__ __forceinline__ f32x4_t load_f32x4(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, AUX));
}
template <int AUX>
__device__ __forceinline__ uint32_t load_u32(rsrc_t r, uint32_t byte_off) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, AUX);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return v;
}
template <int AUX>
__device__ __forceinline__ void store_u32(rsrc_t r, uint32_t byte_off, uint32_t v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)byte_off, 0, AUX);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
template <int AUX>
__device__ __forceinline__ void store_f32x4(rsrc_t r, uint32_t byte_off, const f32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)byte_off, 0, AUX);
}
// The T exchange of an XCD: plain stores and L1-bypassing loads through the
// XCD's L2 when the workgroup placement is verified (`local`), device-
// coherent accesses otherwise.
__device__ __forceinline__ void xstore_f32(bool local, rsrc_t r, uint32_t off, float v) {
  if (local) store_f32<0>(r, off, v); else store_f32<kCoherent>(r, off, v);
}
__device__ __forceinline__ void xstore_f32x4(bool local, rsrc_t r, uint32_t off, const f32x4_t& v) {
  if (local) store_f32x4<0>(r, off, v); else store_f32x4<kCoherent>(r, off, v);
}
__device__ __forceinline__ void xstore_u32(bool local, rsrc_t r, uint32_t off, uint32_t v) {
  if (local) store_u32<0>(r, off, v); else store_u32<kCoherent>(r, off, v);
}
__device__ __forceinline__ f32x4_t xload_f32x4(bool local, rsrc_t r, uint32_t off) {
  return local ? load_f32x4<kSkipL1>(r, off) : load_f32x4<kCoherent>(r, off);
}
__device__ __forceinline__ uint32_t xload_u32(bool local, rsrc_t r, uint32_t off) {
  return local ? load_u32<kSkipL1>(r, off) : load_u32<kCoherent>(r, off);
}

__device__ __forceinline__ int opq(int v) {
  asm volatile("" : "+s"(v));
  return v;
}
__device__ __forceinline__ uint64_t opq64(uint64_t v) {
  asm volatile("" : "+s"(v));
  return v;
}
template <class T>
__device__ __forceinline__ T* opqp(T* p) {
  return (T*)opq64((uint64_t)p);
}
__device__ __forceinline__ XcdProj opaque_proj(const XcdProj& s) {
  XcdProj P;
  P.A = opqp(s.A);
  P.B = opqp(s.B);
  P.Y = opqp(s.Y);
  P.ctrl = opqp(s.ctrl);
  P.err = opqp(s.err);
  P.flags = opqp(s.flags);
  P.tpart = opqp(s.tpart);
  P.tfin = opqp(s.tfin);
  P.ypart = opqp(s.ypart);
  P.r = opq(s.r);
  P.N = opq(s.N);
  P.p0 = opq(s.p0);
  P.pn = opq(s.pn);
  P.pa = opq(s.pa);
  P.rs = opq(s.rs);
  P.nc = opq(s.nc);
  P.cpr_a = opq(s.cpr_a);
  P.cpr_b = opq(s.cpr_b);
  P.da = opq(s.da);
  P.db = opq(s.db);
  P.ldtp = opq(s.ldtp);
  P.ws = opq(s.ws);
  P.stall_xor = (uint32_t)opq((int)s.stall_xor);
  return P;
}

// Raise the timeout flags of projection p (device word and host word).
__device__ __forceinline__ void raise_timeout(const XcdProj& P) { raise_stall(P.ctrl, P.err); }

// One wave spins until the `count` words of `r` at word offsets
// first + stride * i (i < count <= 64) all equal `want`.  Gives up after
// `limit` rounds, raising the timeout flags.
__device__ __forceinline__ void spin_flags(const XcdProj& P, rsrc_t r, int first, int stride, int count,
                                           uint32_t want, bool local, uint32_t limit, int lane) {
  uint32_t spins = 0;
  while (true) {
    bool ok = true;
    if (lane < count) ok = xload_u32(local, r, (uint32_t)(first + stride * lane) * 4u) == want;
    if (__all(ok)) break;
    if (++spins > limit) {
      if (lane == 0) raise_timeout(P);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
}


}  // namespace

__device__ __forceinline__ uint32_t udiv(uint32_t a, uint32_t b) { return a / b; }

__global__ __launch_bounds__(kXThreads) void lr_decode_xcd_kernel(const XcdArgs a) {
  extern __shared__ __align__(16) char xl[];
  const int tid = threadIdx.x;
  const int w = __builtin_amdgcn_readfirstlane(tid >> 6);
  const int l = tid & 63;
  const int wg = blockIdx.x;
  const int x = wg & 7, i = wg >> 3;
  int pi = 0;
#pragma unroll
  for (int t = 1; t < kXcdMaxProj; ++t)
    if (t < a.nproj && i >= a.p[t].p0) pi = t;
  // this projection's arguments, held in registers for the whole kernel (read
  // through an opaque copy: otherwise the compiler reloads them from the
  // argument segment inside the loops, and every such scalar load makes the
  // next LDS wait also wait for memory)
  const XcdProj P = opaque_proj(a.p[pi]);
  const int il = i - P.p0;                  // workgroup within the projection on this XCD
  const int M = opq(a.M), K = opq(a.K), r = P.r, N = P.N;
  const uint16_t* const Xp = (const uint16_t*)opq64((uint64_t)a.X);
  const int mq = (M + 3) >> 2;              // 4-row quads of T and Y in the exchange tables
  const bool two = M > 8;                   // T as two operand planes (hi, lo) instead of one packed plane
  const int pb = P.pn - P.pa;

  const uint32_t gen = __builtin_amdgcn_readfirstlane(ld_agent_u32(P.ctrl));
  const uint32_t epoch = gen + 1u == 0u ? 1u : gen + 1u;
  uint64_t tr[16] = {};
  XT(0);

  // rank range of this XCD (all products below stay far inside 32 bits:
  // every matrix is below 2 GiB)
  const int R0 = (int)(((uint32_t)x * (uint32_t)r) >> 3), R1 = (int)(((uint32_t)(x + 1) * (uint32_t)r) >> 3);
  const int RW = R1 - R0;
  const int nks = (K + 31) >> 5;
  const int nks2 = (RW + 31) >> 5;          // rank k-steps of GEMM2
  const int ldt = 32 * ((((r + 7) >> 3) + 31) >> 5) + 8;  // T plane row (elements), for the widest range

  const rsrc_t rX = make_rsrc(Xp, (int64_t)M * K * 2);
  const rsrc_t rA = make_rsrc(P.A, (int64_t)K * r * 2);
  const rsrc_t rB = make_rsrc(P.B, (int64_t)r * N * 2);
  const bool loc = opq(a.xcd_local) != 0;
  const uint32_t spin_limit = (uint32_t)opq((int)a.spin_limit);
  const int colb = 16 * mq;                 // bytes per column of an exchange table
  const int lgrs = 31 - __builtin_clz((unsigned)P.rs);  // rs is a power of two
  const int ks = P.pa >> lgrs;
  const rsrc_t rTP = make_rsrc(P.tpart, (int64_t)8 * ks * P.ldtp * colb);
  const rsrc_t rTF = make_rsrc(P.tfin, (int64_t)8 * P.ldtp * colb);
  const rsrc_t rYP = make_rsrc(P.ypart, (int64_t)8 * pb * P.ws * colb);
  const rsrc_t rFL = make_rsrc(P.flags, (int64_t)3 * 8 * P.pn * 4);
  const int fl1 = 0, fl2 = 8 * P.pn, fl3 = 16 * P.pn;  // word offsets of the three flag arrays
  const int lane_col = l & 15, lane_q = l >> 4;         // accumulator lane -> column, row quad

  f32x4_t acc[kXcdTilesA > kXcdTilesB ? kXcdTilesA : kXcdTilesB];
#pragma unroll
  for (int g = 0; g < (kXcdTilesA > kXcdTilesB ? kXcdTilesA : kXcdTilesB); ++g) acc[g] = zero4();

  if (il < P.pa) {
    // ============================================================ A workgroup
    // (sub-range rho, K slab kap): partial T of rank columns [c0, c1) over
    // the slab's k-steps; wave w takes k-steps s_lo + w, s_lo + w + 8, ...
    const int ia = il, rho = (int)udiv((uint32_t)ia, (uint32_t)ks), kap = ia - rho * ks;
    const int c0 = R0 + ((rho * RW) >> lgrs), c1 = R0 + (((rho + 1) * RW) >> lgrs);
    const int W = c1 - c0;
    const int s_lo = (int)udiv((uint32_t)(kap * nks), (uint32_t)ks);
    const int s_hi = (int)udiv((uint32_t)((kap + 1) * nks), (uint32_t)ks);
    // LDS rows of cpr_a + 1 chunks: the odd pitch keeps the transposing
    // reads of rows 8 apart off the same banks (the pad chunk is not loaded)
    const int rp = P.cpr_a + 1, ninst = (32 * rp + 63) >> 6;
    const int tile_a = 1024 * ninst, slot_a = tile_a + 1024, row_a = rp * 16;
    char* const ring = xl + w * P.da * slot_a;
    const int na = s_hi - s_lo > w ? (s_hi - s_lo - w + 7) >> 3 : 0;
    const int lpk = ninst + 1;              // A DMA instructions per k-step + the X tile
    const int ng1 = (W + 15) >> 4;
    int rr[kXcdMaxInst], cc[kXcdMaxInst];   // lane -> (row, chunk) of each A instruction of a k-step
    tile_lanes<kXcdMaxInst>(rp, l, rr, cc);
    uint32_t aoff[kXcdMaxInst];             // byte offset of each lane's chunk in k-step 0 (row 0 = A row 0)
    bool aok[kXcdMaxInst];
#pragma unroll
    for (int u = 0; u < kXcdMaxInst; ++u) {
      aok[u] = u < ninst && rr[u] < 32 && cc[u] < P.cpr_a && 8 * cc[u] < W;
      aoff[u] = 2u * ((uint32_t)rr[u] * (uint32_t)r + (uint32_t)(c0 + 8 * cc[u]));
    }
    const uint32_t kstep_bytes = 64u * (uint32_t)r;  // 32 rows of A
    const int xm = l >> 2, xc = l & 3;      // X tile: lane -> row xm, chunk xc (16 x 32 elements)
    const uint32_t xoff = 2u * ((uint32_t)xm * (uint32_t)K + 8u * (uint32_t)xc);
    // the wave holding the last element of A (row K - 1, column r - 1) or of
    // X (row M - 1, column K - 1) patches it (see the header)
    const int s_last = nks - 1;
    const bool has_last_k = s_last >= s_lo + w && s_last < s_hi && ((s_last - s_lo - w) & 7) == 0;
    const bool patch_a = has_last_k && c1 == r && W > 0;
    const uint32_t a_last = patch_a ? scalar_elem(P.A, (int64_t)K * r - 1) : 0u;
    const uint32_t x_last = has_last_k ? scalar_elem(Xp, (int64_t)M * K - 1) : 0u;
    auto issue = [&](int t, int slot_i) {
      const int s = s_lo + w + 8 * t;
      char* slot = ring + slot_i * slot_a;
      const uint32_t base = (uint32_t)s * kstep_bytes;
      const int krem = K - 32 * s;          // rows of this k-step inside A
#pragma unroll
      for (int u = 0; u < kXcdMaxInst; ++u)
        if (u < ninst) dma16(rA, slot + 1024 * u, aok[u] && rr[u] < krem ? base + aoff[u] : kXOut);
      const bool xok = xm < M && 32 * s + 8 * xc < K;
      dma16(rX, slot + tile_a, xok ? xoff + 64u * (uint32_t)s : kXOut);
    };
    const int pre = na < P.da ? na : P.da;
    for (int t = 0; t < pre; ++t) issue(t, t);
    XT(1);
    const int m = l & 15, kq = l >> 4;
    int slot_i = 0;
    for (int t = 0; t < na; ++t) {
      const int s = s_lo + w + 8 * t;
      const int ahead = (na - 1 - t) < (P.da - 1) ? (na - 1 - t) : (P.da - 1);
      wait_vm_dyn(ahead * lpk);
      char* slot = ring + slot_i * slot_a;
      if (s == s_last && l == 0) {
        if (patch_a)  // element (K - 1, r - 1): row K - 1 - 32 s, column r - 1 - c0 of the piece
          *reinterpret_cast<uint16_t*>(slot + (K - 1 - 32 * s) * row_a + (r - 1 - c0) * 2) = (uint16_t)a_last;
        // element (M - 1, K - 1) of X: row M - 1, column K - 1 - 32 s of the X tile
        *reinterpret_cast<uint16_t*>(slot + tile_a + (M - 1) * 64 + (K - 1 - 32 * s) * 2) = (uint16_t)x_last;
      }
      wait_lds();
      // X operand: row m, columns 32 s + 8 kq .. + 7 (past K: cleared)
      u32x4_t xo = *reinterpret_cast<const u32x4_t*>(slot + tile_a + m * 64 + kq * 16);
      xo = mask_cols(xo, 32 * s + 8 * kq, K);
#pragma unroll
      for (int g0 = 0; g0 < kXcdTilesA; g0 += 4) {
        if (g0 < ng1) {
          u32x4_t bo[4];
          tr_operands<4>(slot, row_a, g0, l, bo);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (g0 + u < ng1) {
              const u32x4_t b = 16 * (g0 + u) + lane_col < W ? bo[u] : zerou4();
              acc[g0 + u] = mfma_16x16x32(xo, b, acc[g0 + u]);
            }
          }
        }
      }
      if (t + P.da < na) {
        wait_lds();  // this slot's reads are done before the next k-step's loads overwrite it
        issue(t + P.da, slot_i);
      }
      slot_i = slot_i + 1 == P.da ? 0 : slot_i + 1;
    }
    XT(2);
    // the eight waves' partials of every tile into their own ring regions
    // (lane-major: lane l's four rows of column l % 16)
    {
      f32x4_t* red = reinterpret_cast<f32x4_t*>(ring);
#pragma unroll
      for (int g = 0; g < kXcdTilesA; ++g)
        if (g < ng1) red[g * 64 + l] = acc[g];
    }
    barrier_all();
    // wave w sums tiles g = w, w + 8, ... over the waves in wave order and
    // stores them into this (XCD, K-slab) row of the partial-T table:
    // column c0 - R0 + 16 g + l % 16, rows 4 (l / 16) .. + 3
    const uint32_t trow = (uint32_t)((x * ks + kap) * P.ldtp + (c0 - R0)) * (uint32_t)colb;
    for (int g = w; g < ng1; g += 8) {
      f32x4_t v = zero4();
#pragma unroll
      for (int ww = 0; ww < 8; ++ww) {
        const f32x4_t pv = reinterpret_cast<const f32x4_t*>(xl + ww * P.da * slot_a)[g * 64 + l];
        v[0] += pv[0]; v[1] += pv[1]; v[2] += pv[2]; v[3] += pv[3];
      }
      const int col = 16 * g + lane_col;
      const bool ok = lane_q < mq && col < W;
      xstore_f32x4(loc, rTP, ok ? trow + (uint32_t)(col * colb + 16 * lane_q) : kXOut, v);
    }
    XT(9);
    wait_vmem_all();  // the partial is visible before its flag
    XT(10);
    barrier_all();
    if (w == 0 && l == 0) xstore_u32(loc, rFL, (uint32_t)(fl1 + x * P.pa + ia) * 4u, epoch);
    XT(3);
    // every partial of the XCD's A workgroups is in: this one sums columns
    // [ia RW / pa, (ia + 1) RW / pa) of the range over the ks slabs in slab
    // order (lane = column, rows in quads) and publishes them
    if (w == 0) spin_flags(P, rFL, fl1 + x * P.pa, 1, P.pa, epoch ^ P.stall_xor, loc, spin_limit, l);
    barrier_all();
    XT(4);
    {
      const int e0 = (int)udiv((uint32_t)(ia * RW), (uint32_t)P.pa);
      const int e1 = (int)udiv((uint32_t)((ia + 1) * RW), (uint32_t)P.pa);
      for (int col = e0 + tid; col < e1; col += kXThreads) {
        for (int qq = 0; qq < mq; ++qq) {
          f32x4_t v = zero4();
          for (int k0 = 0; k0 < ks; k0 += 8) {
            f32x4_t pv[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              const uint32_t off = (uint32_t)(((x * ks + k0 + u) * P.ldtp + col) * colb + 16 * qq);
              pv[u] = xload_f32x4(loc, rTP, k0 + u < ks ? off : kXOut);
            }
#pragma unroll
            for (int u = 0; u < 8; ++u) {
              v[0] += pv[u][0]; v[1] += pv[u][1]; v[2] += pv[u][2]; v[3] += pv[u][3];
            }
          }
          xstore_f32x4(loc, rTF, (uint32_t)((x * P.ldtp + col) * colb + 16 * qq), v);
        }
      }
    }
    wait_vmem_all();
    barrier_all();
    if (w == 0 && l == 0) xstore_u32(loc, rFL, (uint32_t)(fl2 + x * P.pa + ia) * 4u, epoch);
    XT(5);
  } else {
    // ============================================================ B workgroup
    // column slab [n0, n1) of the projection over this XCD's rank range;
    // wave w takes column chunk w % nc and the rank k-steps t = w / nc,
    // w / nc + 8 / nc, ...
    const int ib = il - P.pa;
    const int n0 = (int)udiv((uint32_t)(ib * N), (uint32_t)pb), n1 = (int)udiv((uint32_t)((ib + 1) * N), (uint32_t)pb);
    const int sw = n1 - n0;
    const int lgnc = 31 - __builtin_clz((unsigned)P.nc);  // nc is a power of two
    const int nkc = 8 >> lgnc, ch = w & (P.nc - 1), kc = w >> lgnc;
    const int cb0 = n0 + ((ch * sw) >> lgnc), cb1 = n0 + (((ch + 1) * sw) >> lgnc);
    const int WB = cb1 - cb0;
    const int ng2 = (WB + 15) >> 4;
    const int nb = nks2 > kc ? (nks2 - kc + nkc - 1) >> (3 - lgnc) : 0;
    const int rp = P.cpr_b + 1, ninst = (32 * rp + 63) >> 6;  // padded LDS rows, as for A
    const int slot_b = 1024 * ninst, row_b = rp * 16;
    char* const ring = xl + w * P.db * slot_b;
    char* const lds_t = xl + 8 * P.db * slot_b;
    int rr[kXcdMaxInst], cc[kXcdMaxInst];
    tile_lanes<kXcdMaxInst>(rp, l, rr, cc);
    uint32_t boff[kXcdMaxInst];             // byte offset of each lane's chunk in local k-step 0
    bool bok[kXcdMaxInst];
#pragma unroll
    for (int u = 0; u < kXcdMaxInst; ++u) {
      bok[u] = u < ninst && rr[u] < 32 && cc[u] < P.cpr_b && 8 * cc[u] < WB;
      boff[u] = 2u * ((uint32_t)(R0 + rr[u]) * (uint32_t)N + (uint32_t)(cb0 + 8 * cc[u]));
    }
    const uint32_t kstep_bytes = 64u * (uint32_t)N;  // 32 rows of B
    // the wave holding B's last element (row r - 1, column N - 1) patches it
    const int t_last = nks2 - 1;
    const bool patch_b = R1 == r && RW > 0 && cb1 == N && WB > 0 && nb > 0 && ((t_last - kc) & (nkc - 1)) == 0;
    const uint32_t b_last = patch_b ? scalar_elem(P.B, (int64_t)r * N - 1) : 0u;
    auto issue = [&](int u2, int slot_i) {
      const int t = kc + nkc * u2;
      char* slot = ring + slot_i * slot_b;
      const uint32_t base = (uint32_t)t * kstep_bytes;
      const int jrem = RW - 32 * t;         // rows of this k-step inside the range
#pragma unroll
      for (int u = 0; u < kXcdMaxInst; ++u)
        if (u < ninst) dma16(rB, slot + 1024 * u, bok[u] && rr[u] < jrem ? base + boff[u] : kXOut);
    };
    const int pre = nb < P.db ? nb : P.db;
    for (int u2 = 0; u2 < pre; ++u2) issue(u2, u2);
    XT(1);
#ifdef LR_DECODE_TRACE
    wait_vmem_all();
    XT(9);
#endif
    // T of the XCD's rank range, published by its A workgroups: the MFMA
    // operand plane(s) (M <= 8: rows 0-7 bf16 hi of T rows 0-7, rows 8-15
    // lo; otherwise plane 0 hi and plane 1 lo of rows 0-15), zero past M and
    // past the range.  Wave 0 polls (its own loads are counted first, so the
    // first k-steps of B land before the poll can complete)
    if (w == 0) spin_flags(P, rFL, fl2 + x * P.pa, 1, P.pa, epoch, loc, spin_limit, l);
    barrier_all();
    XT(2);
    {
      uint16_t* tp = reinterpret_cast<uint16_t*>(lds_t);
      const int lgq = two ? 2 : 1;          // row quads of T held in the plane(s): 4 or 2
      const int ncol = 32 * nks2;
      for (int it = tid; it < (ncol << lgq); it += kXThreads) {
        const int j = it >> lgq, qq = it & ((1 << lgq) - 1);
        f32x4_t v = zero4();
        if (j < RW && qq < mq) v = xload_f32x4(loc, rTF, (uint32_t)((x * P.ldtp + j) * colb + 16 * qq));
#pragma unroll
        for (int u = 0; u < 4; ++u) {
          const int mm = 4 * qq + u;
          const float f = mm < M ? v[u] : 0.f;
          const uint32_t hb = f32_to_bf16_rne(f);
          const uint32_t lb = f32_to_bf16_rne(f - __uint_as_float(hb << 16));
          tp[mm * ldt + j] = (uint16_t)hb;
          tp[((two ? 16 : 8) + mm) * ldt + j] = (uint16_t)lb;
        }
      }
    }
    barrier_all();
    XT(3);
    const uint16_t* tp = reinterpret_cast<const uint16_t*>(lds_t);
    int slot_i = 0;
    for (int u2 = 0; u2 < nb; ++u2) {
      const int t = kc + nkc * u2;
      const int ahead = (nb - 1 - u2) < (P.db - 1) ? (nb - 1 - u2) : (P.db - 1);
      wait_vm_dyn(ahead * ninst);
      char* slot = ring + slot_i * slot_b;
      if (patch_b && t == t_last && l == 0)
        *reinterpret_cast<uint16_t*>(slot + (r - 1 - R0 - 32 * t) * row_b + (N - 1 - cb0) * 2) = (uint16_t)b_last;
      wait_lds();
      const u32x4_t t0 = *reinterpret_cast<const u32x4_t*>(tp + (l & 15) * ldt + 32 * t + 8 * (l >> 4));
      u32x4_t t1 = zerou4();
      if (two) t1 = *reinterpret_cast<const u32x4_t*>(tp + (16 + (l & 15)) * ldt + 32 * t + 8 * (l >> 4));
#pragma unroll
      for (int g0 = 0; g0 < kXcdTilesB; g0 += 4) {
        if (g0 < ng2) {
          u32x4_t bo[4];
          tr_operands<4>(slot, row_b, g0, l, bo);
#pragma unroll
          for (int u = 0; u < 4; ++u) {
            if (g0 + u < ng2) {
              const u32x4_t bb = 16 * (g0 + u) + lane_col < WB ? bo[u] : zerou4();
              acc[g0 + u] = mfma_16x16x32(t0, bb, acc[g0 + u]);
              if (two) acc[g0 + u] = mfma_16x16x32(t1, bb, acc[g0 + u]);
            }
          }
        }
      }
      if (u2 + P.db < nb) {
        wait_lds();
        issue(u2 + P.db, slot_i);
      }
      slot_i = slot_i + 1 == P.db ? 0 : slot_i + 1;
    }
    XT(4);
    // this wave's partials (M <= 8: output rows m and m + 8, T hi and lo,
    // add up) into its own ring region, lane-major
    {
      f32x4_t* red = reinterpret_cast<f32x4_t*>(ring);
#pragma unroll
      for (int g = 0; g < kXcdTilesB; ++g) {
        if (g < ng2) {
          f32x4_t v = acc[g];
          if (!two) {
#pragma unroll
            for (int u = 0; u < 4; ++u) v[u] += __shfl_xor(v[u], 32);
          }
          red[g * 64 + l] = v;
        }
      }
    }
    barrier_all();
    // wave w sums tiles g = kc, kc + nkc, ... of its chunk over the chunk's
    // nkc waves in wave order and stores the partial Y (device-coherent: the
    // other XCDs read it): slab column cb0 - n0 + 16 g + l % 16, rows
    // 4 (l / 16) .. + 3
    const int qy = x * pb + ib;
    const uint32_t yrow = (uint32_t)(qy * P.ws + (cb0 - n0)) * (uint32_t)colb;
    for (int g = kc; g < ng2; g += nkc) {
      f32x4_t v = zero4();
      for (int k2 = 0; k2 < nkc; ++k2) {
        const f32x4_t pv = reinterpret_cast<const f32x4_t*>(xl + (ch + P.nc * k2) * P.db * slot_b)[g * 64 + l];
        v[0] += pv[0]; v[1] += pv[1]; v[2] += pv[2]; v[3] += pv[3];
      }
      const int col = 16 * g + lane_col;
      const bool ok = lane_q < mq && (two || l < 32) && col < WB;
      store_f32x4<kCoherent>(rYP, ok ? yrow + (uint32_t)(col * colb + 16 * lane_q) : kXOut, v);
    }
    wait_vmem_all();
    barrier_all();
    XT(5);
    // across the XCDs: this workgroup sums the x-th eighth of its slab's
    // columns over the eight XCDs' partials, in XCD order, and stores bf16 Y
    if (w == 0) {
      if (l == 0) store_u32<kCoherent>(rFL, (uint32_t)(fl3 + qy) * 4u, epoch);
      spin_flags(P, rFL, fl3 + ib, pb, 8, epoch, false, spin_limit, l);
    }
    barrier_all();
    XT(6);
    const int e0 = (x * sw) >> 3, e1 = ((x + 1) * sw) >> 3;
    const rsrc_t rY = make_rsrc(P.Y, (int64_t)M * N * 2);
    const int qq = tid & 3;                 // lane = (column, row quad)
    for (int col = e0 + (tid >> 2); col < e1 && qq < mq; col += kXThreads / 4) {
      f32x4_t pv[8];
#pragma unroll
      for (int xx = 0; xx < 8; ++xx)
        pv[xx] = load_f32x4<kCoherent>(rYP, (uint32_t)(((xx * pb + ib) * P.ws + col) * colb + 16 * qq));
      f32x4_t v = zero4();
#pragma unroll
      for (int xx = 0; xx < 8; ++xx) {
        v[0] += pv[xx][0]; v[1] += pv[xx][1]; v[2] += pv[xx][2]; v[3] += pv[xx][3];
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int mm = 4 * qq + u;
        store_u16(rY, mm < M ? 2u * ((uint32_t)mm * (uint32_t)N + (uint32_t)(n0 + col)) : kXOut,
                  f32_to_bf16_rne(v[u]));
      }
    }
  }
  XT(7);
  // count this workgroup out once every read of this launch's exchanges is done
  wait_vmem_all();
  barrier_all();
  XT(8);
  if (tid == 0) {
    const uint32_t done = __hip_atomic_fetch_add(P.ctrl + 1, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if (done + 1u == (uint32_t)(8 * P.pn)) {
      st_agent_u32(P.ctrl + 1, 0u);
      st_agent_u32(P.ctrl, epoch);
    }
  }
#ifdef LR_DECODE_TRACE
  if (a.trace && tid == 0)
    for (int t = 0; t < 16; ++t) a.trace[((int64_t)(epoch & 1) * gridDim.x + wg) * 16 + t] = tr[t];
#else
  (void)tr;
#endif
}

// DMA instructions per k-step of a tile with cpr chunks per row (padded pitch).
static int xcd_inst(int cpr) { return (32 * (cpr + 1) + 63) >> 6; }

hipError_t launch_decode_xcd(const XcdArgs& a, int lds_bytes, hipStream_t stream) {
  static std::atomic<uint64_t> attr_done{0};
  if (a.M < 1 || a.M > 16 || a.nproj < 1 || a.nproj > kXcdMaxProj || a.K < 1 || lds_bytes < 1 ||
      lds_bytes > kXcdMaxLds)
    return hipErrorInvalidValue;
  int total = 0;
  for (int t = 0; t < a.nproj; ++t) {
    const XcdProj& P = a.p[t];
    if (P.p0 != total || P.pn < 2 || P.pa < 1 || P.pa >= P.pn || P.rs < 1 || P.pa % P.rs != 0 ||
        !(P.nc == 1 || P.nc == 2 || P.nc == 4 || P.nc == 8) || P.cpr_a < 2 || P.cpr_a > 2 * kXcdTilesA ||
        (P.cpr_a & 1) || P.cpr_b < 2 || P.cpr_b > 2 * kXcdTilesB || (P.cpr_b & 1) || P.da < 1 || P.db < 1 ||
        P.da * (xcd_inst(P.cpr_a) + 1) > 62 || P.db * xcd_inst(P.cpr_b) > 62 || P.ldtp < (P.r + 7) / 8 ||
        (int64_t)P.ws * (P.pn - P.pa) < P.N || !P.A || !P.B || !P.Y || !P.ctrl || !P.flags || !P.tpart || !P.tfin ||
        !P.ypart)
      return hipErrorInvalidValue;
    total += P.pn;
  }
  if (total * 8 != a.grid) return hipErrorInvalidValue;
  static std::atomic<uint64_t> occ{0};
  hipError_t e = ensure_dynamic_lds((const void*)lr_decode_xcd_kernel, kXcdMaxLds, attr_done);
  if (e == hipSuccess) e = check_coresident((const void*)lr_decode_xcd_kernel, kXThreads, (size_t)lds_bytes, a.grid, occ);
  if (e != hipSuccess || a.check_only) return e;
  hipLaunchKernelGGL(lr_decode_xcd_kernel, dim3((unsigned)a.grid), dim3(kXThreads), (size_t)lds_bytes, stream, a);
  return hipGetLastError();
}

int decode_xcd_blocks_per_cu(int lds_bytes) {
  int n = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, (const void*)lr_decode_xcd_kernel, kXThreads, (size_t)lds_bytes) !=
      hipSuccess)
    return 0;
  return n;
}

}  // namespace lrk
