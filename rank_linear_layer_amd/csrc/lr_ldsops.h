// LDS helpers shared by the decode kernels that stream row-major factors
// straight into LDS (direct-to-LDS buffer loads) and read MFMA operands back
// with the gfx950 transposing LDS read.
#pragma once

#include "lr_device.h"

namespace lrk {

typedef __attribute__((address_space(3))) void* lds_ptr_t;

// Wave-uniform n in [0, 63]: wait until at most n of this wave's vector
// memory operations are outstanding.
__device__ __forceinline__ void wait_vm_dyn(int n) {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
#define LR_VM_CASE(c) \
  case c: __builtin_amdgcn_s_waitcnt(((c) & 15) | (((c) >> 4) << 14) | 0x0F70); break;
  switch (n) {
    LR_VM_CASE(0) LR_VM_CASE(1) LR_VM_CASE(2) LR_VM_CASE(3) LR_VM_CASE(4) LR_VM_CASE(5) LR_VM_CASE(6)
    LR_VM_CASE(7) LR_VM_CASE(8) LR_VM_CASE(9) LR_VM_CASE(10) LR_VM_CASE(11) LR_VM_CASE(12) LR_VM_CASE(13)
    LR_VM_CASE(14) LR_VM_CASE(15) LR_VM_CASE(16) LR_VM_CASE(17) LR_VM_CASE(18) LR_VM_CASE(19) LR_VM_CASE(20)
    LR_VM_CASE(21) LR_VM_CASE(22) LR_VM_CASE(23) LR_VM_CASE(24) LR_VM_CASE(25) LR_VM_CASE(26) LR_VM_CASE(27)
    LR_VM_CASE(28) LR_VM_CASE(29) LR_VM_CASE(30) LR_VM_CASE(31) LR_VM_CASE(32) LR_VM_CASE(33) LR_VM_CASE(34)
    LR_VM_CASE(35) LR_VM_CASE(36) LR_VM_CASE(37) LR_VM_CASE(38) LR_VM_CASE(39) LR_VM_CASE(40) LR_VM_CASE(41)
    LR_VM_CASE(42) LR_VM_CASE(43) LR_VM_CASE(44) LR_VM_CASE(45) LR_VM_CASE(46) LR_VM_CASE(47) LR_VM_CASE(48)
    LR_VM_CASE(49) LR_VM_CASE(50) LR_VM_CASE(51) LR_VM_CASE(52) LR_VM_CASE(53) LR_VM_CASE(54) LR_VM_CASE(55)
    LR_VM_CASE(56) LR_VM_CASE(57) LR_VM_CASE(58) LR_VM_CASE(59) LR_VM_CASE(60) LR_VM_CASE(61) LR_VM_CASE(62)
    default: break;
  }
#undef LR_VM_CASE
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// Wait for this wave's LDS operations (lgkmcnt = 0), nothing else.
__device__ __forceinline__ void wait_lds() {
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
  __builtin_amdgcn_s_waitcnt(0xC07F);
  __atomic_signal_fence(__ATOMIC_SEQ_CST);
}

// All eight waves meet; LDS writes before it are visible after it.  Vector
// memory operations still in flight stay in flight.
__device__ __forceinline__ void barrier_all() { barrier_lds(); }

__device__ __forceinline__ void dma16(rsrc_t r, char* lds_wave_base, uint32_t byte_off) {
  __builtin_amdgcn_raw_ptr_buffer_load_lds(r, (lds_ptr_t)lds_wave_base, 16, (int)byte_off, 0, 0, 0);
}

// Lane l's 32 x 16 MFMA operands from a row-major tile in LDS (rows of
// row_bytes, 8-byte aligned) for NT column tiles: operand t holds rows
// 8 (l / 16) .. + 7 of column 16 (g0 + t) + l % 16, read with the
// transposing LDS read (within a 16-lane group, lane 4 q + c reads row q at
// columns 4 c .. 4 c + 3 and receives one column of the 4 x 16 tile).
// One asm block issues every read and then waits for them: the compiler
// cannot tell these reads from the direct-to-LDS loads still in flight into
// other slots, and left to itself it would wait for every one of those.
template <int NT>
__device__ __forceinline__ void tr_operands(const char* tile, int row_bytes, int g0, int l, u32x4_t (&op)[NT]) {
  const int kq = l >> 4, q = (l >> 2) & 3, c = l & 3;
  const char* p = tile + (8 * kq + q) * row_bytes + (32 * g0 + 8 * c);
  const uint32_t a0 = (uint32_t)(uintptr_t)(__attribute__((address_space(3))) const char*)p;
  const uint32_t a1 = a0 + 4u * (uint32_t)row_bytes;
  typedef uint32_t u32x2_t __attribute__((ext_vector_type(2)));
  u32x2_t lo[NT], hi[NT];
  if constexpr (NT == 4) {
    asm volatile(
        "ds_read_b64_tr_b16 %0, %8\n\t"
        "ds_read_b64_tr_b16 %1, %9\n\t"
        "ds_read_b64_tr_b16 %2, %8 offset:32\n\t"
        "ds_read_b64_tr_b16 %3, %9 offset:32\n\t"
        "ds_read_b64_tr_b16 %4, %8 offset:64\n\t"
        "ds_read_b64_tr_b16 %5, %9 offset:64\n\t"
        "ds_read_b64_tr_b16 %6, %8 offset:96\n\t"
        "ds_read_b64_tr_b16 %7, %9 offset:96\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0]), "=&v"(lo[1]), "=&v"(hi[1]), "=&v"(lo[2]), "=&v"(hi[2]), "=&v"(lo[3]),
          "=&v"(hi[3])
        : "v"(a0), "v"(a1)
        : "memory");
  } else {
    static_assert(NT == 1, "1 or 4 tiles per read batch");
    asm volatile(
        "ds_read_b64_tr_b16 %0, %2\n\t"
        "ds_read_b64_tr_b16 %1, %3\n\t"
        "s_waitcnt lgkmcnt(0)"
        : "=&v"(lo[0]), "=&v"(hi[0])
        : "v"(a0), "v"(a1)
        : "memory");
  }
#pragma unroll
  for (int t = 0; t < NT; ++t) op[t] = u32x4_t{lo[t][0], lo[t][1], hi[t][0], hi[t][1]};
}


// Lane -> (row, chunk) of the DMA instructions of a k-step tile with rp
// chunks per LDS row: instruction u covers flat chunks 64 u .. 64 u + 63.
// Filled incrementally (one division per lane, not one per instruction).
template <int NI>
__device__ __forceinline__ void tile_lanes(int rp, int l, int (&rr)[NI], int (&cc)[NI]) {
  int row = l / rp, col = l - row * rp;
  const int q64 = 64 / rp, r64 = 64 - q64 * rp;
#pragma unroll
  for (int u = 0; u < NI; ++u) {
    rr[u] = row;
    cc[u] = col;
    col += r64;
    row += q64;
    if (col >= rp) {
      col -= rp;
      ++row;
    }
  }
}

}  // namespace lrk
