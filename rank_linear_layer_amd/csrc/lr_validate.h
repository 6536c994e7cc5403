// Argument validation and work partitioning of the C ABI.  Pure host C++
// with no HIP dependency, so it is unit-tested on the CPU (g++), and the
// same code runs inside the library.
#pragma once

#include <stdint.h>
#include <stdio.h>

#include <algorithm>

#include "../../include/lr_linear.h"

namespace lrv {

constexpr int kDecodeMaxM = LR_DECODE_MAX_M;

struct Range {
  uintptr_t lo, hi;  // [lo, hi)
};

inline Range span(const void* p, int64_t elems) {
  uintptr_t a = (uintptr_t)p;
  return Range{a, a + (uintptr_t)(elems > 0 ? elems : 0) * 2u};
}
inline bool overlaps(Range a, Range b) { return a.lo < b.hi && b.lo < a.hi && a.lo != a.hi && b.lo != b.hi; }
inline bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Largest dimension accepted; keeps every flat index well inside int64 and
// every per-row index inside int32.
constexpr int64_t kMaxDim = (int64_t)1 << 24;
// Kernels address each matrix through a 32-bit buffer range.
constexpr int64_t kMaxMatrixBytes = ((int64_t)1 << 31) - 64;

inline lr_status check_create(int64_t K, int64_t r, int64_t N, const void* A, const void* B, int64_t max_M,
                              uint32_t flags, char* err, size_t errlen) {
  if (!A || !B) { snprintf(err, errlen, "A and B must be non-null device pointers"); return LR_ERR_INVALID_ARG; }
  if (K < 1 || r < 1 || N < 1) {
    snprintf(err, errlen, "K, r and N must be >= 1 (got K=%lld r=%lld N=%lld)", (long long)K, (long long)r, (long long)N);
    return LR_ERR_INVALID_ARG;
  }
  if (K > kMaxDim || r > kMaxDim || N > kMaxDim || max_M > kMaxDim) {
    snprintf(err, errlen, "dimension above the supported maximum %lld", (long long)kMaxDim);
    return LR_ERR_INVALID_ARG;
  }
  if (max_M < 0) { snprintf(err, errlen, "max_M must be >= 0 (got %lld)", (long long)max_M); return LR_ERR_INVALID_ARG; }
  if (!aligned16(A) || !aligned16(B)) { snprintf(err, errlen, "A and B must be 16-byte aligned"); return LR_ERR_INVALID_ARG; }
  if (K * r * 2 > kMaxMatrixBytes || r * N * 2 > kMaxMatrixBytes || max_M * K * 2 > kMaxMatrixBytes ||
      max_M * N * 2 > kMaxMatrixBytes || max_M * ((r + 31) / 32 * 32) * 2 > kMaxMatrixBytes) {
    snprintf(err, errlen, "a matrix would exceed 2 GiB (32-bit buffer addressing)");
    return LR_ERR_UNSUPPORTED;
  }
  const uint32_t known = LR_FLAG_FORCE_DECODE | LR_FLAG_FORCE_PREFILL | LR_FLAG_DECODE_STREAMING |
                         LR_FLAG_PREFILL_TWO_WAVE | LR_FLAG_PREFILL_ONE_WAVE | LR_FLAG_DENSE | LR_FLAG_FACTORED |
                         LR_FLAG_DECODE_SPLIT | LR_FLAG_DECODE_RESIDENT | LR_FLAG_DECODE_XCD | LR_FLAG_TEST_STALL;
  if (flags & ~known) { snprintf(err, errlen, "unknown flag bits 0x%x", flags & ~known); return LR_ERR_UNSUPPORTED; }
  if ((flags & LR_FLAG_FORCE_DECODE) && (flags & LR_FLAG_FORCE_PREFILL)) {
    snprintf(err, errlen, "FORCE_DECODE and FORCE_PREFILL are exclusive");
    return LR_ERR_INVALID_ARG;
  }
  if ((flags & LR_FLAG_PREFILL_TWO_WAVE) && (flags & LR_FLAG_PREFILL_ONE_WAVE)) {
    snprintf(err, errlen, "PREFILL_TWO_WAVE and PREFILL_ONE_WAVE are exclusive");
    return LR_ERR_INVALID_ARG;
  }
  {
    const uint32_t dk =
        flags & (LR_FLAG_DECODE_STREAMING | LR_FLAG_DECODE_SPLIT | LR_FLAG_DECODE_RESIDENT | LR_FLAG_DECODE_XCD);
    if (dk & (dk - 1)) {
      snprintf(err, errlen, "DECODE_STREAMING, DECODE_SPLIT, DECODE_RESIDENT and DECODE_XCD are exclusive");
      return LR_ERR_INVALID_ARG;
    }
  }
  if ((flags & LR_FLAG_DECODE_SPLIT) && (max_M > kDecodeMaxM || (flags & LR_FLAG_FORCE_PREFILL))) {
    // its decode reads a copy of A and B made at create; a handle that also
    // ran prefill would read the live factors there and the copy here
    snprintf(err, errlen, "DECODE_SPLIT handles are decode-only: max_M must be <= %d and FORCE_PREFILL unset",
             (int)kDecodeMaxM);
    return LR_ERR_INVALID_ARG;
  }
  if ((flags & LR_FLAG_DENSE) && (flags & LR_FLAG_FACTORED)) {
    snprintf(err, errlen, "DENSE and FACTORED are exclusive");
    return LR_ERR_INVALID_ARG;
  }
  if ((flags & LR_FLAG_DENSE) && K * N * 2 > kMaxMatrixBytes) {
    snprintf(err, errlen, "DENSE: W = A.B (%lld x %lld) would exceed 2 GiB", (long long)K, (long long)N);
    return LR_ERR_UNSUPPORTED;
  }
  if ((flags & LR_FLAG_FORCE_DECODE) && max_M > kDecodeMaxM) {
    snprintf(err, errlen, "FORCE_DECODE needs max_M <= %d (got %lld)", kDecodeMaxM, (long long)max_M);
    return LR_ERR_UNSUPPORTED;
  }
  return LR_OK;
}

// Dense fallback choice: forced by a flag, else taken when the factors hold
// at least 95% of the bytes of the K x N matrix they replace (the
// factorization then saves almost no HBM traffic, and one GEMM without a T
// hand-off is faster) and W is addressable through a 32-bit range.
constexpr int64_t kDensePercent = 95;
inline bool choose_dense(int64_t K, int64_t r, int64_t N, uint32_t flags) {
  if (flags & LR_FLAG_FACTORED) return false;
  if (flags & LR_FLAG_DENSE) return true;
  if (K * N * 2 > kMaxMatrixBytes) return false;
  return 100 * r * (K + N) >= kDensePercent * K * N;
}

struct Shape {
  int64_t K, r, N, max_M;
  const void* A;
  const void* B;
};

inline lr_status check_run(const Shape& s, const void* X, const void* Y, int64_t M, char* err, size_t errlen) {
  if (M < 0 || M > s.max_M) {
    snprintf(err, errlen, "M=%lld outside [0, max_M=%lld]", (long long)M, (long long)s.max_M);
    return LR_ERR_INVALID_ARG;
  }
  if (M == 0) return LR_OK;
  if (!X || !Y) { snprintf(err, errlen, "X and Y must be non-null device pointers"); return LR_ERR_INVALID_ARG; }
  if (!aligned16(X) || !aligned16(Y)) { snprintf(err, errlen, "X and Y must be 16-byte aligned"); return LR_ERR_INVALID_ARG; }
  const Range ry = span(Y, M * s.N);
  if (overlaps(ry, span(X, M * s.K)) || overlaps(ry, span(s.A, s.K * s.r)) || overlaps(ry, span(s.B, s.r * s.N))) {
    snprintf(err, errlen, "Y overlaps an input (X, A or B)");
    return LR_ERR_INVALID_ARG;
  }
  return LR_OK;
}

// Projections sharing X in one call: 1..kMaxGroup handles of equal K, each
// run checked as lr_linear_run would check it, no output overlapping another
// output or another projection's factors.
constexpr int kMaxGroup = LR_GROUP_MAX;
inline lr_status check_group(const Shape* s, int n, const void* X, const void* const* Ys, int64_t M, char* err,
                             size_t errlen) {
  if (n < 1 || n > kMaxGroup) {
    snprintf(err, errlen, "n=%d projections; 1 to %d share X in one call", n, kMaxGroup);
    return LR_ERR_INVALID_ARG;
  }
  for (int i = 1; i < n; ++i)
    if (s[i].K != s[0].K) {
      snprintf(err, errlen, "projection %d has K=%lld, projection 0 has K=%lld", i, (long long)s[i].K,
               (long long)s[0].K);
      return LR_ERR_INVALID_ARG;
    }
  for (int i = 0; i < n; ++i) {
    const lr_status st = check_run(s[i], X, Ys[i], M, err, errlen);
    if (st != LR_OK) return st;
  }
  if (M == 0) return LR_OK;
  for (int i = 0; i < n; ++i) {
    const Range ri = span(Ys[i], M * s[i].N);
    for (int j = 0; j < n; ++j) {
      if (j == i) continue;
      if (j > i && overlaps(ri, span(Ys[j], M * s[j].N))) {
        snprintf(err, errlen, "outputs %d and %d overlap", i, j);
        return LR_ERR_INVALID_ARG;
      }
      if (overlaps(ri, span(s[j].A, s[j].K * s[j].r)) || overlaps(ri, span(s[j].B, s[j].r * s[j].N))) {
        snprintf(err, errlen, "output %d overlaps the factors of projection %d", i, j);
        return LR_ERR_INVALID_ARG;
      }
    }
  }
  return LR_OK;
}

inline lr_status check_packed(const Shape& g, const Shape& u, const void* X, const void* Yg, const void* Yu, int64_t M,
                              char* err, size_t errlen) {
  const Shape s[2] = {g, u};
  const void* Ys[2] = {Yg, Yu};
  return check_group(s, 2, X, Ys, M, err, errlen);
}

// ------------------------------------------------------------ partition ---
// Decode kernels cut the rank into Jw slices and K and N into S slices;
// workgroup (js, s) owns rank slice js, K slice s and N slice s.
//  kind 1 (LDS-resident): Jw is a multiple of 8 and slices are at most 128
//    columns wide (a multiple of 8); every slab of a workgroup fits in LDS at
//    once: at most 8 k-tiles of 32 rows and 2 n-tiles of 128 columns; one
//    workgroup per CU, so Jw * S <= CUs.  Requires K % 8 == 0 (rows of X are
//    staged as aligned 16-byte chunks).
//  kind 0 (streaming, 120-wide slices): any shape; tiles stream through
//    registers.
// S minimises the elements streamed by the busiest workgroup (ties to the
// smaller S), subject to Jw * S <= budget.
struct DecPart {
  int kind, Jw, S, ktps, ntps, js_w, nt_w;
  int ga, gn, gb, gpw;  // kinds 2 and 3
  int g, nt;            // kinds 3 and 4: workgroups; kind 3: column groups per T producer
  int maxc;             // kind 4: contributors per rank slice
};

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int64_t round_up8(int64_t a) { return (a + 7) / 8 * 8; }

inline bool decode_resident_partition(int64_t K, int64_t r, int64_t N, int budget, DecPart* out) {
  if (K % 8 != 0) return false;
  const int64_t kt = 32, nt = 128;
  // Jw a multiple of 8 (one rank-slice group per XCD slot), slices <= 128 wide
  const int64_t Jw = 8 * ceil_div(ceil_div(r, 128), 8);
  const int64_t js_w = round_up8(ceil_div(r, Jw));
  const int64_t nk = ceil_div(K, kt), nn = ceil_div(N, nt);
  int64_t best_s = -1, best_cost = -1;
  for (int64_t S = 1; S * Jw <= budget; ++S) {
    const int64_t ktps = ceil_div(nk, S), ntps = ceil_div(nn, S);
    if (ktps > 8 || ntps > 2) continue;
    if ((S - 1) * ktps >= nk && (S - 1) * ntps >= nn) continue;  // a fully idle slice
    const int64_t cost = ktps * kt * js_w + ntps * js_w * nt;
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_s = S; }
  }
  if (best_s < 0) return false;
  out->kind = 1;
  out->Jw = (int)Jw;
  out->S = (int)best_s;
  out->ktps = (int)ceil_div(nk, best_s);
  out->ntps = (int)ceil_div(nn, best_s);
  out->js_w = (int)js_w;
  out->nt_w = (int)nt;
  return true;
}

inline DecPart decode_streaming_partition(int64_t K, int64_t r, int64_t N, int budget) {
  const int64_t js_w = 120, kt = 32, nt = 120;
  DecPart p{};
  p.kind = 0;
  p.js_w = (int)js_w;
  p.nt_w = (int)nt;
  p.Jw = (int)ceil_div(r, js_w);
  const int64_t nk = ceil_div(K, kt), nn = ceil_div(N, nt);
  int64_t smax = budget / p.Jw;
  if (smax < 1) smax = 1;
  const int64_t useful = nk > nn ? nk : nn;
  if (smax > useful) smax = useful;
  int64_t best_s = 1, best_cost = -1;
  for (int64_t S = 1; S <= smax; ++S) {
    const int64_t cost = ceil_div(nk, S) * kt * js_w + ceil_div(nn, S) * js_w * nt;  // elements per WG
    if (best_cost < 0 || cost < best_cost) { best_cost = cost; best_s = S; }
  }
  p.S = (int)best_s;
  p.ktps = (int)ceil_div(nk, best_s);
  p.ntps = (int)ceil_div(nn, best_s);
  return p;
}

// kind 2 (role-split): GA = ceil(r/16) workgroups each produce 16 rank
//   columns of T over all of K; GB workgroups each produce gpw 16-column
//   groups of Y (gpw the smallest of 1, 2, 4, 8 that fits) over the whole
//   rank, holding their B blocks in registers: at most max_blocks 1 KB
//   blocks per wave, eight waves, so ceil(ceil(r/32) / (8 / gpw)) <=
//   max_blocks.  GA + GB <= budget (one launch, every workgroup resident),
//   the decode layout of B below 2 GiB (32-bit offsets), and T's GEMM2
//   operand planes (one plane of 16 x (32 ceil(r/32) + 8) bf16 for
//   max_M <= 8, two otherwise; whole kilobytes) within max_t_bytes of LDS.
inline bool decode_split_partition(int64_t K, int64_t r, int64_t N, int budget, DecPart* out, int max_blocks = 16,
                                   int64_t max_M = 16, int64_t max_t_bytes = 144 * 1024) {
  const int64_t ga = ceil_div(r, 16), gn = ceil_div(N, 16), nkb = ceil_div(r, 32);
  if (gn * nkb * 1024 >= ((int64_t)1 << 31) || ceil_div(K, 32) * 1024 >= ((int64_t)1 << 31)) return false;
  if (ceil_div((max_M > 8 ? 2 : 1) * 16 * (32 * nkb + 8) * 2, 1024) * 1024 > max_t_bytes) return false;
  for (int gpw = 1; gpw <= 8; gpw *= 2) {
    const int64_t gb = ceil_div(gn, gpw);
    const int64_t per = ceil_div(nkb, 8 / gpw);
    if (ga + gb <= budget && per <= max_blocks) {
      out->kind = 2;
      out->Jw = (int)ga;  // reported as the producer counts
      out->S = 1;
      out->ktps = (int)ceil_div(K, 32);
      out->ntps = (int)per;
      out->js_w = 16;
      out->nt_w = 16 * gpw;
      out->ga = (int)ga;
      out->gn = (int)gn;
      out->gb = (int)gb;
      out->gpw = gpw;
      return true;
    }
  }
  return false;
}

// kind 3 (role-split, streaming Y): for shapes whose B does not fit the
//   Y producers' registers (the MLP projections).  G = min(budget,
//   GA + GN) workgroups all compute Y; the first GA (GA = ceil(r/16) <= G)
//   first produce T and so take fewer column groups: bytes per workgroup
//   are balanced with A's slab plus X (ceil(K/32) KB + max_M K 2 bytes) per
//   T producer against ceil(r/32) KB of B per column group; a T producer's
//   slab above the average share rules the kind out.  Every wave
//   holds at most max_blocks of a group's B blocks (twice) and as many T
//   operands (twice for max_M > 8, allowed up to 8 blocks per wave).
inline bool decode_split_stream_partition(int64_t K, int64_t r, int64_t N, int budget, DecPart* out,
                                          int max_blocks = 16, int64_t max_M = 16) {
  const int64_t ga = ceil_div(r, 16), gn = ceil_div(N, 16), nkb = ceil_div(r, 32), nka = ceil_div(K, 32);
  const int64_t per = ceil_div(nkb, 8);
  if (per > max_blocks || (max_M > 8 && per > 8)) return false;
  if (gn * nkb * 1024 >= ((int64_t)1 << 31) || nka * 1024 >= ((int64_t)1 << 31)) return false;
  if (ga > budget) return false;
  const int64_t g = budget < ga + gn ? budget : ga + gn;
  const int64_t gy = g - ga;
  const double ca = (double)nka + (double)(max_M * K * 2) / 1024.0, cb = (double)nkb;
  int64_t nt;
  if (gy == 0) {
    nt = ceil_div(gn, ga);
  } else {
    const double target = ((double)ga * ca + (double)gn * cb) / (double)g;
    // a T producer's slab heavier than the average workgroup's share would
    // make the T side the bound (the down projection: K = 14336): the
    // slice-split kernels spread A over every workgroup instead
    if (ca > target) return false;
    nt = (int64_t)((target - ca) / cb);
    if (ga * nt > gn) nt = gn / ga;
  }
  out->kind = 3;
  out->Jw = (int)ga;
  out->S = 1;
  out->ktps = (int)nka;
  out->ntps = (int)per;
  out->js_w = 16;
  out->nt_w = 16;
  out->ga = (int)ga;
  out->gn = (int)gn;
  out->gb = (int)gy;
  out->gpw = 0;
  out->g = (int)g;
  out->nt = (int)nt;
  return true;
}

// kind 4 (role-split, flat): for A-heavy shapes that neither split kind
//   takes (the down projection).  G = budget workgroups each take an equal
//   share of A's operand blocks in slice-major order (GA <= G, so a share
//   spans at most two slices) and an equal share of Y's column groups; a
//   slice's first contributor adds the others' partials (at most
//   ceil(nkA / floor(TB / G)) + 1 contributors, TB = GA ceil(K/32) >= G so
//   that no share is empty).
//   Y work as in kind 3.
inline bool decode_split_flat_partition(int64_t K, int64_t r, int64_t N, int budget, DecPart* out,
                                        int max_blocks = 16, int64_t max_M = 16) {
  const int64_t ga = ceil_div(r, 16), gn = ceil_div(N, 16), nkb = ceil_div(r, 32), nka = ceil_div(K, 32);
  const int64_t per = ceil_div(nkb, 8);
  if (per > max_blocks || (max_M > 8 && per > 8)) return false;
  const int64_t tb = ga * nka;
  if (gn * nkb * 1024 >= ((int64_t)1 << 31) || tb * 1024 >= ((int64_t)1 << 31)) return false;
  // every workgroup needs a non-empty share: an owner waits for each
  // workgroup id between it and the slice's last contributor
  if (ga > budget || budget < 1 || tb < budget) return false;
  const int64_t rlen = tb / budget;
  out->kind = 4;
  out->Jw = (int)ga;
  out->S = 1;
  out->ktps = (int)nka;
  out->ntps = (int)per;
  out->js_w = 16;
  out->nt_w = 16;
  out->ga = (int)ga;
  out->gn = (int)gn;
  out->gb = budget - (int)ga;
  out->gpw = 0;
  out->g = budget;
  out->nt = 0;
  out->maxc = (int)(ceil_div(nka, rlen) + 1);
  return true;
}

// `split`: take a role-split kind when one fits (else the others).
inline DecPart decode_partition(int64_t K, int64_t r, int64_t N, int budget, bool allow_resident = true,
                                bool split = false, int64_t max_M = 16) {
  DecPart p{};
  if (split && decode_split_partition(K, r, N, budget, &p, 16, max_M)) return p;
  if (split && decode_split_stream_partition(K, r, N, budget, &p, 16, max_M)) return p;
  if (split && decode_split_flat_partition(K, r, N, budget, &p, 16, max_M)) return p;
  if (allow_resident && decode_resident_partition(K, r, N, budget, &p)) return p;
  return decode_streaming_partition(K, r, N, budget);
}

inline int64_t round_up(int64_t a, int64_t b) { return ceil_div(a, b) * b; }

// XCD-sliced decode (the default decode kernel, lr_decode_xcd.hip).  With
// P workgroups per XCD (one per compute unit), a projection given pn of
// them per XCD: XCD x owns rank rows [x r / 8, (x + 1) r / 8).  The first pa
// of its pn workgroups stream A: (pa / rs) K-slabs x rs rank sub-ranges,
// each computing a partial T; the other pb = pn - pa stream B, one column
// slab of N each, for GEMM2 over the XCD's rank range.  A compute unit that
// streams one factor never holds the exchange of the other behind its own
// requests.  pa follows the bytes each side streams (A and X against B).
// Wide row pieces stream best (a compute unit moves whole 128-byte lines
// much faster than pieces of a few dozen bytes): rs is the smallest power of
// two that keeps a sub-range within kXcdMaxTilesA 16-column MFMA tiles, and
// a slab is cut into nc (1, 2, 4 or 8) column chunks of at most
// kXcdMaxTilesB tiles.  The k-steps in flight per wave (da, db) are as many
// as the LDS holds and each wave's vector-memory counter (6 bits) counts.
constexpr int kXcdMaxTilesA = 16;
constexpr int kXcdMaxTilesB = 16;
constexpr int64_t kXcdLdsBytes = 160 * 1024;
constexpr int kXcdMaxInFlight = 62;         // vector-memory operations a wave keeps in flight
struct XcdPlan {
  int pn, pa, rs, nc;
  int cpr_a, cpr_b;  // 16-byte chunks per LDS row of an A piece / a B chunk
  int da, db;        // k-steps in flight per wave of an A / a B workgroup
  int ldtp, ws;      // rank-range and slab lengths of the exchange tables
  int64_t lds;       // dynamic LDS bytes (the larger of the two roles)
  int64_t tpart_bytes, tfin_bytes, ypart_bytes;
};
inline bool xcd_plan(int64_t K, int64_t r, int64_t N, int pn, int64_t max_M, XcdPlan* out) {
  if (pn < 2 || K < 1 || r < 1 || N < 1 || max_M < 1 || max_M > kDecodeMaxM) return false;
  const int64_t rw = ceil_div(r, 8);          // widest XCD rank range
  const int64_t nks = ceil_div(K, 32);
  int rs = 1;
  while (ceil_div(rw, rs) > 16 * kXcdMaxTilesA && rs < pn) rs *= 2;
  if (ceil_div(rw, rs) > 16 * kXcdMaxTilesA) return false;
  // A workgroups in proportion to the bytes streamed, a multiple of rs,
  // leaving at least one B workgroup
  const double abytes = (double)K * (double)r + (double)max_M * (double)K * 8.0;
  const double bbytes = (double)r * (double)N;
  int pa = (int)((double)pn * abytes / (abytes + bbytes) / rs + 0.5) * rs;
  if (pa < rs) pa = rs;
  while (pa > pn - 1 && pa > rs) pa -= rs;
  if (pa > pn - 1) return false;
  XcdPlan p{};
  p.pn = pn;
  p.pa = pa;
  p.rs = rs;
  const int64_t ks = pa / rs;
  p.cpr_a = (int)(2 * ceil_div(ceil_div(rw, rs), 16));
  p.ws = (int)ceil_div(N, pn - pa);
  p.nc = 1;
  while (ceil_div(p.ws, p.nc) > 16 * kXcdMaxTilesB && p.nc < 8) p.nc *= 2;
  if (ceil_div(p.ws, p.nc) > 16 * kXcdMaxTilesB) return false;
  p.cpr_b = (int)(2 * ceil_div(ceil_div(p.ws, p.nc), 16));
  const int64_t nks2 = ceil_div(rw, 32);
  const int64_t ldt = 32 * nks2 + 8;
  const int64_t tbytes = (max_M > 8 ? 32 : 16) * ldt * 2;
  // LDS tiles have rows of cpr + 1 chunks (an odd pitch spreads rows over
  // the banks), loaded by whole 64-lane instructions
  const int64_t ia = ceil_div(32 * (p.cpr_a + 1), 64), ib = ceil_div(32 * (p.cpr_b + 1), 64);
  const int64_t slot_a = 1024 * ia + 1024, slot_b = 1024 * ib;
  const int64_t ka = std::max<int64_t>(1, ceil_div(ceil_div(nks, ks), 8));   // k-steps of the busiest A wave
  const int64_t kb = std::max<int64_t>(1, ceil_div(nks2, 8 / p.nc));        // and of the busiest B wave
  const int64_t da_max = std::min<int64_t>(ka, kXcdMaxInFlight / (ia + 1));
  const int64_t db_max = std::min<int64_t>(kb, kXcdMaxInFlight / ib);
  if (da_max < 1 || db_max < 1 || 8 * slot_a > kXcdLdsBytes || 8 * slot_b + tbytes > kXcdLdsBytes) return false;
  int64_t da = 1, db = 1;
  while (da < da_max && 8 * (da + 1) * slot_a <= kXcdLdsBytes) ++da;
  while (db < db_max && 8 * (db + 1) * slot_b + tbytes <= kXcdLdsBytes) ++db;
  p.da = (int)da;
  p.db = (int)db;
  p.ldtp = (int)rw;
  p.lds = std::max<int64_t>(8 * da * slot_a, 8 * db * slot_b + tbytes);
  const int64_t colb = 16 * ceil_div(max_M, 4);
  p.tpart_bytes = 8 * ks * p.ldtp * colb;
  p.tfin_bytes = 8 * (int64_t)p.ldtp * colb;
  p.ypart_bytes = 8 * (int64_t)(pn - pa) * p.ws * colb;
  *out = p;
  return true;
}

// Prefill launch plan: tile width 32 * nb columns and a k-split.  Cost
// unit: about 0.14 us.  A launch takes as many rounds as it has workgroups
// per compute unit.  A k-split (splits > 1) adds a reduction kernel: one
// launch (about 14 units) plus writing and reading the fp32 partials (about
// 700 KB per unit).  The cheapest plan wins (fewer splits, then the wider
// tile, on a tie).
struct PrePlan {
  int nb, splits, split_steps;
  int kind;     // 0: two waves per SIMD, tile 256 x 32 nb; 1: one wave per SIMD, tile 256 x 256
  double cost;  // the model's cost of the plan
};
// Kernel, tile width and k-split for one prefill phase, from a cost model in
// units of about 0.14 us: rounds of the 256-CU machine times (k-steps per
// split x the kernel's per-step cost + its per-tile cost: start-up,
// epilogue), plus the partial write/read and reduction launch when k is
// split.  Per 32-deep k-step of one tile, measured on MI355X from kernel
// traces (MLP up-projection M = 4096: phase 1 at nb = 6, one round of 128
// steps, 106 us; phase 2 at nb = 7, four rounds of 90 steps, 325 us; the
// one-wave kernel 156 and 432 us; X . W at K = N = 4096 with nb = 4, two
// rounds of 128 steps, 165 us, and one-wave, one round, 151 us; nb = 2 and
// 3 scaled from the same phases with only that width allowed): two-wave
// nb = 2 3.6, 3 4.0, 4 4.6, 6 6.0, 7 6.4, 40 per tile (80 with fp32
// partials); one-wave 8.3, 85 per tile (200 with fp32 partials), k-splits on
// 64-deep stages.  No cost depends on the weight's leading dimension (r or N) modulo
// 8: both kernels read misaligned rows with the same instructions as
// aligned ones.  `kinds`: bit 0 allows the two-wave kernel, bit 1 the
// one-wave kernel (which needs a 16-byte aligned P: X with K mod 8 = 0, or
// T).
constexpr int kPlanTwoWave = 1;
constexpr int kPlanOneWave = 2;
inline PrePlan prefill_plan(int64_t rows, const int64_t* out_cols, int nout, int64_t kd, int num_cus,
                            int max_splits = 32, int kinds_allowed = kPlanTwoWave) {
  const int64_t row_tiles = ceil_div(rows, 256);
  const int64_t nks = ceil_div(kd, 32);
  const int cus = num_cus > 0 ? num_cus : 1;
  int64_t cols = 0;
  for (int i = 0; i < nout; ++i) cols += out_cols[i];
  PrePlan best{7, 1, (int)nks, 0, 0.0};
  double best_cost = -1;
  const struct {
    int nb, kind;
    double per_step, per_tile, per_tile_split;
  } kinds[6] = {{8, 1, 8.3, 85.0, 200.0}, {7, 0, 6.4, 40.0, 80.0}, {6, 0, 6.0, 40.0, 80.0},
                {4, 0, 4.6, 40.0, 80.0},    {3, 0, 4.0, 40.0, 80.0},  {2, 0, 3.6, 40.0, 80.0}};
  for (const auto& kn : kinds) {
    if (!(kinds_allowed & (kn.kind == 1 ? kPlanOneWave : kPlanTwoWave))) continue;
    const int gran = kn.kind == 1 ? 2 : 1;
    const int64_t units = ceil_div(nks, gran);
    int64_t tiles = 0;
    for (int i = 0; i < nout; ++i) tiles += row_tiles * ceil_div(out_cols[i], 32 * kn.nb);
    for (int64_t want = 1; want <= max_splits && want <= units; ++want) {
      const int64_t per = ceil_div(units, want);
      const int64_t splits = ceil_div(units, per);  // no empty split
      if (splits != want) continue;
      const int64_t steps = per * gran;
      const int64_t rounds = ceil_div(tiles * splits, cus);
      double cost = (double)rounds * ((double)steps * kn.per_step + (splits > 1 ? kn.per_tile_split : kn.per_tile));
      if (splits > 1) cost += 14.0 + (double)(2 * splits * rows * cols * 4 + rows * cols * 2) / 700e3;
      if (best_cost < 0 || cost < best_cost - 1e-9) {
        best_cost = cost;
        best = PrePlan{kn.nb, (int)splits, (int)steps, kn.kind, cost};
      }
    }
  }
  return best;
}

// fp32 partial bytes a handle needs for its own output over every M <= max_M
// (both phases share the region; M steps of 256 change the tiling).
// For a dense-fallback handle the one GEMM is X . W (N columns, depth K).
inline int64_t prefill_partial_bytes(int64_t max_M, int64_t K, int64_t r_pad, int64_t N, int num_cus,
                                     bool dense = false) {
  // Within one 256-row bucket the tiling is fixed and larger M only makes
  // splitting costlier, so the split count at the bucket's smallest M times
  // its largest M bounds every M in the bucket.
  int64_t need = 0;
  for (int64_t m = 256;; m += 256) {
    const int64_t hi = m < max_M ? m : max_M;
    const int64_t lo = m - 255 < hi ? m - 255 : hi;
    const int64_t c1 = r_pad, c2 = N;
    for (int kinds = 1; kinds <= 3; ++kinds) {
      const int64_t cd = dense ? c2 : c1;
      const PrePlan p1 = prefill_plan(lo, &cd, 1, K, num_cus, 32, kinds);
      const PrePlan p2 = prefill_plan(lo, &c2, 1, dense ? K : r_pad, num_cus, 32, kinds);
      const int64_t n1 = p1.splits > 1 ? p1.splits * hi * round_up(cd, 4) * 4 : 0;
      const int64_t n2 = p2.splits > 1 ? p2.splits * hi * round_up(c2, 4) * 4 : 0;
      need = need > n1 ? need : n1;
      need = need > n2 ? need : n2;
    }
    if (hi == max_M) break;
  }
  return need;
}

}  // namespace lrv
