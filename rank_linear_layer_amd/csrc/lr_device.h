// Device-side building blocks shared by the decode and prefill kernels
// (gfx950 / CDNA4, wave64).
//
// Misaligned rows.  A factor stored row-major with an odd leading dimension
// (rank r = 1637, width N = 3999 ...) has rows that start at arbitrary
// 2-byte boundaries.  The page on dimensional misalignment ("Why Smaller Is
// Slower? ...", section 3.3 and Table 4) traces part of the slowdown to
// exactly this: accesses that no longer fill whole memory sectors.  Here
// every global load stays a naturally aligned 16-byte load.  A lane that
// needs the 8 elements [j, j + 8) of a row loads the aligned 16-byte chunk
// holding element j, takes the following chunk from its right-hand
// neighbour lane through a DPP row shift, and funnel-shifts the pair by the
// row's misalignment.  The 16 lanes of a DPP row load 16 consecutive chunks
// and the first 15 of them produce output, so a wave row covers 120
// columns.  Within the tiles used here all rows that one load
// instruction touches have the same misalignment (they are congruent
// mod 8), so the shift is wave-uniform and the selection below is a
// uniform branch.
//
// MFMA operands.  v_mfma_f32_16x16x32_bf16 wants the reduction index
// contiguous inside each lane (8 bf16 per lane).  Weights are stored with
// the *output* index contiguous, so a lane that loaded rows k0..k0+7 at
// columns j..j+7 transposes that 8 x 8 block in registers (v_perm) into
// eight operands, one per column; MFMA e of a group then computes output
// columns {8 * lane16 + e}.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lrk {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4_t __attribute__((ext_vector_type(4)));

__device__ __forceinline__ f32x4_t mfma_16x16x32(const u32x4_t& a, const u32x4_t& b, const f32x4_t& c) {
  return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8_t, a),
                                                 __builtin_bit_cast(bf16x8_t, b), c, 0, 0, 0);
}

__device__ __forceinline__ int64_t min64(int64_t a, int64_t b) { return a < b ? a : b; }
__device__ __forceinline__ f32x4_t zero4() { return f32x4_t{0.f, 0.f, 0.f, 0.f}; }
__device__ __forceinline__ u32x4_t zerou4() { return u32x4_t{0u, 0u, 0u, 0u}; }

// bf16 bits -> fp32
__device__ __forceinline__ float bf16_lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16_hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

// fp32 -> bf16 bits, round to nearest even (inputs finite).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// Lane i of each 16-lane DPP row receives `src` of lane i + 1; lane 15 of
// each row keeps `old`.
__device__ __forceinline__ uint32_t dpp_row_shl1(uint32_t old, uint32_t src) {
  return (uint32_t)__builtin_amdgcn_update_dpp((int)old, (int)src, 0x101, 0xf, 0xf, false);
}
__device__ __forceinline__ u32x4_t dpp_row_shl1(const u32x4_t& old, const u32x4_t& src) {
  u32x4_t r;
  r[0] = dpp_row_shl1(old[0], src[0]);
  r[1] = dpp_row_shl1(old[1], src[1]);
  r[2] = dpp_row_shl1(old[2], src[2]);
  r[3] = dpp_row_shl1(old[3], src[3]);
  return r;
}

// Elements (2i+1, 2i+2) of the pair (y = dword i, x = dword i + 1).
__device__ __forceinline__ uint32_t odd_pair(uint32_t x, uint32_t y) { return (y >> 16) | (x << 16); }

// Elements [d, d + 8) of the 16-element window (lo, hi); d is wave-uniform.
__device__ __forceinline__ u32x4_t realign(const u32x4_t& lo, const u32x4_t& hi, int d) {
  u32x4_t o;
  switch (d) {
    default:
    case 0: o = lo; break;
    case 1: o[0] = odd_pair(lo[1], lo[0]); o[1] = odd_pair(lo[2], lo[1]); o[2] = odd_pair(lo[3], lo[2]); o[3] = odd_pair(hi[0], lo[3]); break;
    case 2: o[0] = lo[1]; o[1] = lo[2]; o[2] = lo[3]; o[3] = hi[0]; break;
    case 3: o[0] = odd_pair(lo[2], lo[1]); o[1] = odd_pair(lo[3], lo[2]); o[2] = odd_pair(hi[0], lo[3]); o[3] = odd_pair(hi[1], hi[0]); break;
    case 4: o[0] = lo[2]; o[1] = lo[3]; o[2] = hi[0]; o[3] = hi[1]; break;
    case 5: o[0] = odd_pair(lo[3], lo[2]); o[1] = odd_pair(hi[0], lo[3]); o[2] = odd_pair(hi[1], hi[0]); o[3] = odd_pair(hi[2], hi[1]); break;
    case 6: o[0] = lo[3]; o[1] = hi[0]; o[2] = hi[1]; o[3] = hi[2]; break;
    case 7: o[0] = odd_pair(hi[0], lo[3]); o[1] = odd_pair(hi[1], hi[0]); o[2] = odd_pair(hi[2], hi[1]); o[3] = odd_pair(hi[3], hi[2]); break;
  }
  return o;
}

// Elements [d, d + 8) of the 16-element window (lo, hi), d in 0..7 per lane
// (not wave-uniform: each lane selects its own shift).
__device__ __forceinline__ u32x4_t realign_lane(const u32x4_t& lo, const u32x4_t& hi, int d) {
  const uint32_t w[8] = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
  const int q = d >> 1;
  const uint32_t sh = (uint32_t)(d & 1) * 16u;
  u32x4_t o;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const uint32_t a = q == 0 ? w[i] : q == 1 ? w[i + 1] : q == 2 ? w[i + 2] : w[i + 3];
    const uint32_t b = q == 0 ? w[i + 1] : q == 1 ? w[i + 2] : q == 2 ? w[i + 3] : w[i + 4];
    o[i] = __builtin_amdgcn_alignbit(b, a, sh);
  }
  return o;
}

// Zero the elements of an 8-element segment whose column col0 + e >= ncols.
__device__ __forceinline__ u32x4_t mask_cols(const u32x4_t& v, int64_t col0, int64_t ncols) {
  if (col0 + 8 <= ncols) return v;
  u32x4_t o = zerou4();
#pragma unroll
  for (int p = 0; p < 4; ++p) {
    uint32_t w = v[p];
    uint32_t keep = 0;
    if (col0 + 2 * p < ncols) keep |= 0x0000FFFFu;
    if (col0 + 2 * p + 1 < ncols) keep |= 0xFFFF0000u;
    o[p] = w & keep;
  }
  return o;
}

// 8 x 8 bf16 transpose: seg[q] holds elements (row q, cols 0..7); returns in
// op[e] the 8 rows of column e (row q at vector element q).
__device__ __forceinline__ void transpose8x8(const u32x4_t seg[8], u32x4_t op[8]) {
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const uint32_t sel = (e & 1) ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int p = 0; p < 4; ++p) {
      op[e][p] = __builtin_amdgcn_perm(seg[2 * p + 1][e >> 1], seg[2 * p][e >> 1], sel);
    }
  }
}

// ------------------------------------------------------ buffer loads ---
// All global reads go through buffer resources whose range is the
// matrix itself (rounded up to whole dwords): the hardware returns zero for
// any dword outside it, so tails and overhanging tiles need no branches
// (a branch around a load would make the compiler wait for every load in
// flight at the join).
typedef __amdgpu_buffer_rsrc_t rsrc_t;
constexpr int kRsrcFlags = 0x00020000;  // raw buffer, 32-bit data format
constexpr int kCoherent = 16;           // sc1: device-scope coherent access

__device__ __forceinline__ rsrc_t make_rsrc(const void* base, int64_t bytes) {
  const int64_t rounded = (bytes + 3) & ~(int64_t)3;
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), 0, (int)rounded, kRsrcFlags);
}
// Element e of a bf16 matrix through the scalar cache (wave-uniform e): the
// dword holding it is read whole (it cannot cross a page, so even the 2
// bytes past an odd-length matrix are safe to touch).  Scalar loads are
// counted apart from the vector-memory counter.  Used to patch a matrix's
// last element where an unaligned 16-byte buffer load loses it: the range
// check zeroes every dword that reaches past the range end, and a load that
// starts 2 bytes past a dword boundary puts the last element of a matrix
// ending on a dword boundary into such a dword.
__device__ __forceinline__ uint32_t scalar_elem(const uint16_t* base, int64_t e) {
  const uint64_t byte = (uint64_t)e * 2;
  typedef __attribute__((address_space(4))) const uint32_t* cptr;
  const uint32_t d = *(cptr)((const char*)base + (byte & ~(uint64_t)3));
  return (byte & 2) ? (d >> 16) : (d & 0xFFFFu);
}

__device__ __forceinline__ u32x4_t buf_load16(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(u32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
__device__ __forceinline__ uint32_t buf_load_u16(rsrc_t r, uint32_t byte_off) {
  return (uint32_t)__builtin_amdgcn_raw_buffer_load_b16(r, (int)byte_off, 0, 0);
}
__device__ __forceinline__ f32x4_t buf_load16_coherent(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kCoherent));
}
__device__ __forceinline__ void buf_store16_coherent(rsrc_t r, uint32_t byte_off, const f32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)byte_off, 0, kCoherent);
}
// Loads that skip the compute unit's L1 but may hit the XCD's L2: data
// written by other compute units of the same XCD through that L2.  This is
// the non-temporal bit (nt).  sc0 alone is work-group scope, which may be
// served from a stale L1 line: a poll loop on such a load can spin on the
// old value until the line happens to be evicted.
constexpr int kSkipL1 = 2;
__device__ __forceinline__ f32x4_t buf_load16_l2(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, kSkipL1));
}
// Data written by other compute units of this XCD during this kernel, read
// once: a plain load misses the (kernel-start invalidated) L1 and is served
// by the shared L2.  Only for addresses this compute unit has not read
// before in the kernel.
__device__ __forceinline__ f32x4_t buf_load16_fresh(rsrc_t r, uint32_t byte_off) {
  return __builtin_bit_cast(f32x4_t, __builtin_amdgcn_raw_buffer_load_b128(r, (int)byte_off, 0, 0));
}
__device__ __forceinline__ void buf_store16(rsrc_t r, uint32_t byte_off, const f32x4_t& v) {
  __builtin_amdgcn_raw_buffer_store_b128(__builtin_bit_cast(u32x4_t, v), r, (int)byte_off, 0, 0);
}
// Flag reads for poll loops.  The compiler fences around each load keep it
// inside the loop (a plain buffer load with nothing else touching memory in
// the loop could legally be hoisted out of it).
__device__ __forceinline__ uint32_t buf_load_u32_l2(rsrc_t r, uint32_t byte_off) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kSkipL1);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return v;
}
__device__ __forceinline__ uint32_t buf_load_u32_coherent(rsrc_t r, uint32_t byte_off) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  const uint32_t v = __builtin_amdgcn_raw_buffer_load_b32(r, (int)byte_off, 0, kCoherent);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  return v;
}
__device__ __forceinline__ void buf_store_u32(rsrc_t r, uint32_t byte_off, uint32_t v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)byte_off, 0, 0);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
__device__ __forceinline__ void buf_store_u32_coherent(rsrc_t r, uint32_t byte_off, uint32_t v) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_raw_buffer_store_b32(v, r, (int)byte_off, 0, kCoherent);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}
// Id of the XCD (accelerator complex die) this wave runs on (HW_REG_XCC_ID).
__device__ __forceinline__ uint32_t xcc_id() { return __builtin_amdgcn_s_getreg((15 << 11) | 20) & 0xFu; }

// Raw half of a realigned row-segment load: lane16 of a 16-lane DPP row
// loads the aligned chunk that holds column colbase + 8*lane16 - d of row
// `row` (d = misalignment, see realign_segment).  Lanes 0..14 produce the
// 8 columns [colbase + 8*lane16, +8); lane 15 only supplies the high half
// for lane 14, so one DPP row covers 120 columns.  Rows past the end of
// the matrix read as zero.
__device__ __forceinline__ u32x4_t load_row_raw(rsrc_t r, int64_t row, int64_t ld, int64_t colbase, int lane16) {
  const int64_t c0 = (row * ld + colbase) >> 3;
  return buf_load16(r, (uint32_t)((c0 + lane16) * 16));
}

// Second half: realign the raw chunk with the right-hand neighbour's chunk,
// zero columns >= ncols, and zero the whole segment when !row_ok.  `d` =
// (row * ld + colbase) mod 8 must be uniform over the wave.  Lane 15's
// result is meaningless.
__device__ __forceinline__ u32x4_t realign_segment(const u32x4_t& lo, int d, int64_t col0, int64_t ncols,
                                                   bool row_ok) {
  const u32x4_t hi = dpp_row_shl1(zerou4(), lo);
  const u32x4_t v = mask_cols(realign(lo, hi, d), col0, ncols);
  return row_ok ? v : zerou4();
}

// 8 consecutive elements [k0, k0 + 8) of row `row` of a row-major matrix
// with leading dimension ld (the buffer covers the valid rows).  When ld is
// a multiple of 8 (k0 always is) this is one 16-byte load and the result is
// RAW: columns >= klen are cleared later by kvec_mask, at the point of use,
// so that no instruction touches the destination registers while the load
// is in flight.  Otherwise 8 two-byte loads, masked here (slow path).
__device__ __forceinline__ u32x4_t load_kvec(rsrc_t r, int64_t row, int64_t ld, int64_t k0, int64_t klen,
                                             bool aligned) {
  const int64_t e0 = row * ld + k0;
  if (aligned) return buf_load16(r, (uint32_t)(e0 * 2));
  uint32_t t[8];
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const uint32_t x = buf_load_u16(r, (uint32_t)((e0 + i) * 2));
    t[i] = (k0 + i < klen) ? x : 0u;
  }
  u32x4_t v;
  v[0] = t[0] | (t[1] << 16);
  v[1] = t[2] | (t[3] << 16);
  v[2] = t[4] | (t[5] << 16);
  v[3] = t[6] | (t[7] << 16);
  return v;
}
// Completes load_kvec: with ld and k0 multiples of 8 the segment is either
// entirely inside the row (k0 < klen) or entirely past it.
__device__ __forceinline__ u32x4_t kvec_mask(const u32x4_t& v, int64_t k0, int64_t klen) {
  return (k0 < klen) ? v : zerou4();
}

// Device-coherent (agent scope) relaxed accesses used to exchange partial
// sums between workgroups on different XCDs without L2 write-back or
// invalidate fences: each access bypasses the non-coherent cache state.
__device__ __forceinline__ void st_agent_f32(float* p, float v) {
  __hip_atomic_store(reinterpret_cast<uint32_t*>(p), __float_as_uint(v), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ float ld_agent_f32(const float* p) {
  return __uint_as_float(__hip_atomic_load(reinterpret_cast<const uint32_t*>(p), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT));
}
__device__ __forceinline__ void st_agent_u32(uint32_t* p, uint32_t v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_agent_u32(const uint32_t* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t add_agent_u32(uint32_t* p, uint32_t v) {
  return __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// A cross-workgroup wait gave up: raise the device timeout word ctrl[2] and,
// when the handle has one, the pinned host word `err` (system scope, so the
// host sees it without a device synchronisation).
__device__ __forceinline__ void raise_stall(uint32_t* ctrl, uint32_t* err) {
  st_agent_u32(ctrl + 2, 1u);
  if (err) __hip_atomic_store(err, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_SYSTEM);
}
// Epoch-tagged exchange words between workgroups: {v0, tag, v1, tag}, two
// values of a partial result, each beside a copy of the launch's epoch,
// written as one 16-byte device-coherent store.  A reader that finds the
// epoch it waits for in both tags of a word has both values (each value
// shares an aligned 8-byte half of the store with its tag, and a store is
// never seen split inside such a half), so an exchange needs neither a flag
// nor a wait for the stores to complete: the reader polls the data itself.
__device__ __forceinline__ void xstore_coherent(rsrc_t r, uint32_t off, float v0, float v1, float tag) {
  buf_store16_coherent(r, off, f32x4_t{v0, tag, v1, tag});
}
__device__ __forceinline__ bool xtagged(const f32x4_t& t, uint32_t want) {
  return __float_as_uint(t[1]) == want && __float_as_uint(t[3]) == want;
}
// Polls the exchange word at byte voff of n partials (stride bytes apart
// from base), 16 partials in flight at a time, until all carry `want`, and
// returns the two sums over the partials in order 0 .. n - 1.  A wait that
// reaches spin_limit polls raises the stall words and sums what it read.
__device__ __forceinline__ void xpoll_sum(rsrc_t r, uint32_t base, uint32_t stride, int n, uint32_t voff,
                                          uint32_t want, uint32_t spin_limit, uint32_t* ctrl, uint32_t* err, float& s0,
                                          float& s1) {
  s0 = 0.f;
  s1 = 0.f;
  for (int p0 = 0; p0 < n; p0 += 16) {
    const int np0 = min(16, n - p0);
    f32x4_t t[16];
    uint32_t spins = 0;
    while (true) {
      __atomic_signal_fence(__ATOMIC_SEQ_CST);  // a fresh read every poll
#pragma unroll
      for (int u = 0; u < 16; ++u) t[u] = buf_load16_coherent(r, base + (uint32_t)(p0 + min(u, np0 - 1)) * stride + voff);
      __atomic_signal_fence(__ATOMIC_SEQ_CST);
      bool ok = true;
#pragma unroll
      for (int u = 0; u < 16; ++u) ok = ok && xtagged(t[u], want);
      if (ok) break;
      if (++spins > spin_limit) {
        raise_stall(ctrl, err);
        break;
      }
      __builtin_amdgcn_s_sleep(1);
    }
#pragma unroll
    for (int u = 0; u < 16; ++u)
      if (u < np0) {
        s0 += t[u][0];
        s1 += t[u][2];
      }
  }
}

// Workgroup barrier that orders LDS only: waits for this wave's LDS
// accesses (lgkmcnt = 0) and meets the other waves, without waiting for
// global loads or stores still in flight.  (__syncthreads() also drains the
// vector-memory counter, which would stall every barrier behind loads that
// are deliberately kept in flight and behind write-through stores.)  Code
// that needs global stores or LDS-DMA loads complete calls wait_vmem_all()
// first.
__device__ __forceinline__ void barrier_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);  // vmcnt 63 (no wait), expcnt 7, lgkmcnt 0
  __builtin_amdgcn_s_barrier();
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait until every vector memory operation of this wave has completed
// (gfx9 encoding: vmcnt = 0, expcnt and lgkmcnt left at their maxima).
__device__ __forceinline__ void wait_vmem_all() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0x0F70);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

}  // namespace lrk
