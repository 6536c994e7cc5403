/*
 * lr_gac.h -- rank re-selection for GPU-aligned compression, host side.
 *
 * The constrained-optimization step of GAC ("Why Smaller Is Slower?
 * Dimensional Misalignment in Compressed LLMs", section 4.3, Step 3, with
 * its budget quantization): given each compressible weight's importance
 * score, its parameter cost per retained dimension, the compressor's
 * continuous allocation and a candidate set of dimensions accepted by a
 * latency sweep on the target GPU (section 4.2), pick one candidate per
 * weight that maximizes the sum of score x (parameters kept - parameters
 * at the continuous allocation) within a total parameter budget.  Solved
 * by dynamic programming over the budget on costs quantized by a unit.
 * Pure host code: no GPU, no HIP call.
 */
#ifndef LR_GAC_H
#define LR_GAC_H

#include <stdint.h>

#include "lr_linear.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * lr_gac_select
 *   n          : number of weights (>= 1).
 *   score      : [n] importance scores s_i (any finite value).
 *   unit_cost  : [n] parameters per retained dimension c_i, in [1, 2^31]
 *                (K + N for a rank-d factor pair of a K x N weight; the
 *                row count for a structurally pruned column).
 *   d_star     : [n] the compressor's continuous allocation d*_i.
 *   cand_count : [n] number of candidates of each weight, 1 .. 65535.
 *   cand_dims  : the candidates, weight after weight (sum of cand_count
 *                entries), each in [0, 2^31].
 *   budget     : total parameter budget B (>= 0).
 *   unit       : quantization unit u (> 0), or <= 0 for 8 x min(c_i), the
 *                page's choice for dimensions that are multiples of 8.
 *                Costs are rounded up and the budget down to whole units,
 *                so every selection returned fits the exact budget.
 *   chosen     : [n] out: the selected dimension of each weight.
 *   objective  : out (may be NULL): sum of s_i c_i (d_i - d*_i).
 * Among selections of equal objective the one of smaller quantized cost
 * wins, then the earlier candidates.  All arrays are host memory, borrowed
 * for the call.
 * Errors: INVALID_ARG (null array, n < 1, counts or values out of range,
 * no selection within the budget), UNSUPPORTED (n x (budget / unit + 1)
 * above 2^27 table cells), OUT_OF_MEMORY.
 */
lr_status lr_gac_select(int n, const double* score, const int64_t* unit_cost, const double* d_star,
                        const int* cand_count, const int64_t* cand_dims, int64_t budget, int64_t unit,
                        int64_t* chosen, double* objective);

#ifdef __cplusplus
}
#endif

#endif /* LR_GAC_H */
