// GAC rank re-selection: the constrained-optimization step of "Why Smaller
// Is Slower? Dimensional Misalignment in Compressed LLMs" (section 4.3,
// Step 3: Constrained Optimization, with its budget quantization).
//
// Each compressible weight i has an importance score s_i, a parameter cost
// per retained dimension c_i (K_i + N_i for a rank-d factor pair, the row
// count for a pruned column), the compressor's continuous allocation d*_i,
// and a candidate set C_i of dimensions that the platform sweep accepted
// (section 4.2).  Choosing d_i in C_i costs w = c_i d_i parameters and is
// worth v = s_i (c_i d_i - c_i d*_i); the selection maximizes the total
// value with the total cost within the budget B.  This is a multiple-choice
// knapsack, solved by dynamic programming over the budget:
//     D[i][b] = max_j { D[i-1][b - w'_ij] + v_ij },   D[0][b] = 0,
// on costs and budget quantized by a unit u (the page takes u = 8 times the
// smallest per-dimension cost, since dimensions are multiples of 8):
// w' = ceil(w / u), B' = floor(B / u), so that any selection the table
// admits also fits the exact budget.  Ties go to the smaller total cost,
// then to the earlier candidate, so the result is deterministic.
#include <stdint.h>
#include <stdio.h>
#include <string.h>

#include <new>
#include <vector>

#include "../../include/lr_gac.h"

// defined with the library's error state (lr_last_error)
lr_status lr_internal_fail(lr_status st, const char* msg);

namespace {

constexpr int64_t kMaxTable = (int64_t)1 << 27;  // cells of the choice table (items x budget cells)
constexpr int64_t kMaxValue = (int64_t)1 << 31;  // bound on unit costs and dimensions (products fit 62 bits)

lr_status bad(lr_status st, const char* msg) { return lr_internal_fail(st, msg); }

}  // namespace

extern "C" lr_status lr_gac_select(int n, const double* score, const int64_t* unit_cost, const double* d_star,
                                   const int* cand_count, const int64_t* cand_dims, int64_t budget, int64_t unit,
                                   int64_t* chosen, double* objective) {
  if (n < 1 || !score || !unit_cost || !d_star || !cand_count || !cand_dims || !chosen)
    return bad(LR_ERR_INVALID_ARG, "lr_gac_select: n >= 1 and non-null arrays required");
  if (budget < 0) return bad(LR_ERR_INVALID_ARG, "lr_gac_select: budget must be >= 0");
  int64_t min_cost = 0, total_cands = 0;
  for (int i = 0; i < n; ++i) {
    if (unit_cost[i] < 1 || unit_cost[i] > kMaxValue)
      return bad(LR_ERR_INVALID_ARG, "lr_gac_select: unit costs must be in [1, 2^31]");
    if (cand_count[i] < 1 || cand_count[i] > 65535)
      return bad(LR_ERR_INVALID_ARG, "lr_gac_select: every weight needs 1 to 65535 candidates");
    min_cost = (i == 0 || unit_cost[i] < min_cost) ? unit_cost[i] : min_cost;
    total_cands += cand_count[i];
  }
  for (int64_t k = 0; k < total_cands; ++k)
    if (cand_dims[k] < 0 || cand_dims[k] > kMaxValue)
      return bad(LR_ERR_INVALID_ARG, "lr_gac_select: candidate dimensions must be in [0, 2^31]");
  const int64_t u = unit > 0 ? unit : 8 * min_cost;
  const int64_t Bq = budget / u;
  if ((int64_t)n * (Bq + 1) > kMaxTable)
    return bad(LR_ERR_UNSUPPORTED, "lr_gac_select: the quantized table exceeds 2^27 cells (use a larger unit)");

  // quantized costs and values, item-major
  std::vector<int64_t> wq((size_t)total_cands);
  std::vector<double> val((size_t)total_cands);
  {
    int64_t k = 0;
    for (int i = 0; i < n; ++i)
      for (int j = 0; j < cand_count[i]; ++j, ++k) {
        const int64_t w = unit_cost[i] * cand_dims[k];
        wq[(size_t)k] = (w + u - 1) / u;
        val[(size_t)k] = score[i] * ((double)w - (double)unit_cost[i] * d_star[i]);
      }
  }
  // D over budget cells, rolled; the choice table keeps each item's pick
  // per cell (candidate index + 1, 0 = unreachable)
  const double kNone = -1e300;
  std::vector<double> prev((size_t)(Bq + 1), 0.0), cur((size_t)(Bq + 1));
  std::vector<int64_t> pcost((size_t)(Bq + 1), 0), ccost((size_t)(Bq + 1));
  std::vector<uint16_t> pick;
  try {
    pick.assign((size_t)n * (size_t)(Bq + 1), 0);
  } catch (const std::bad_alloc&) {
    return bad(LR_ERR_OUT_OF_MEMORY, "lr_gac_select: choice table allocation failed");
  }
  int64_t base = 0;
  for (int i = 0; i < n; ++i) {
    for (int64_t b = 0; b <= Bq; ++b) {
      double best = kNone;
      int64_t best_cost = 0;
      int best_j = -1;
      for (int j = 0; j < cand_count[i]; ++j) {
        const int64_t w = wq[(size_t)(base + j)];
        if (w > b || prev[(size_t)(b - w)] == kNone) continue;
        const double v = prev[(size_t)(b - w)] + val[(size_t)(base + j)];
        const int64_t c = pcost[(size_t)(b - w)] + w;
        if (best_j < 0 || v > best || (v == best && c < best_cost)) {
          best = v;
          best_cost = c;
          best_j = j;
        }
      }
      cur[(size_t)b] = best;
      ccost[(size_t)b] = best_cost;
      pick[(size_t)i * (size_t)(Bq + 1) + (size_t)b] = (uint16_t)(best_j + 1);
    }
    prev.swap(cur);
    pcost.swap(ccost);
    base += cand_count[i];
  }
  // the full budget column holds the best over every total cost <= B'
  if (prev[(size_t)Bq] == kNone) return bad(LR_ERR_INVALID_ARG, "lr_gac_select: no selection fits the budget");
  // walk back
  int64_t b = Bq;
  std::vector<int64_t> starts((size_t)n);
  {
    int64_t k = 0;
    for (int i = 0; i < n; ++i) {
      starts[(size_t)i] = k;
      k += cand_count[i];
    }
  }
  double obj = 0;
  for (int i = n - 1; i >= 0; --i) {
    const int j = (int)pick[(size_t)i * (size_t)(Bq + 1) + (size_t)b] - 1;
    if (j < 0) return bad(LR_ERR_INVALID_ARG, "lr_gac_select: inconsistent table");  // unreachable
    const int64_t k = starts[(size_t)i] + j;
    chosen[i] = cand_dims[k];
    obj += val[(size_t)k];
    b -= wq[(size_t)k];
  }
  if (objective) *objective = obj;
  return LR_OK;
}
