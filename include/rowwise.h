/*
 * rowwise.h -- C ABI of the row-wise kernels (gfx950): the row softmax and
 * the fused RMSNorm + SiLU.
 *
 * Row softmax: the TileLang tutorial's row-wise softmax, whose maximum and
 * sum reductions and normalisation stay in registers (pro.edgex.exchange
 * summary, paragraph on the fused epilogue and the row-wise softmax;
 * datastack.it, section "Cosa copre il tutorial"):
 *
 *     y_j = exp(x_j - max_k x_k) / sum_k exp(x_k - max_k x_k)
 *
 * Fused RMSNorm + SiLU: the production kernel of the pages' first summary,
 * RMSNorm and the SiLU activation in one pass (the pages give no formula;
 * the usual RMSNorm with a weight is taken):
 *
 *     z_j = x_j / sqrt(mean_k x_k^2 + eps) * g_j,   y_j = z_j / (1 + exp(-z_j))
 *
 * Both work on R independent rows of length C, row-major [R, C], fp16 or
 * bf16 in and out, fp32 inside; status codes and element types are those of
 * fa.h.
 */
#ifndef ROWWISE_MI355X_H
#define ROWWISE_MI355X_H

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * row_softmax -- enqueue y = softmax(x) along the rows on `stream`.
 *
 * x  device pointer, [R, C] row-major, element `dtype` (2-byte aligned;
 *    16-byte alignment and C % 8 == 0 select the vector path).
 * y  device pointer, [R, C], element `dtype`; written, rounded to nearest
 *    even.  Must not overlap x.
 * R >= 1 (below 2^31), 1 <= C <= 32768 (larger C: FA_ERR_UNSUPPORTED).
 * Checks, ownership and asynchrony as for fa_fwd; NaN inputs make their row
 * NaN.
 */
fa_status row_softmax(const void* x, void* y, int64_t R, int64_t C, int dtype, void* stream);

/*
 * rmsnorm_silu -- enqueue y = silu(rmsnorm(x) * g) along the rows on `stream`.
 *
 * x    device pointer, [R, C] row-major, element `dtype`.
 * g    device pointer, [C], element `dtype`: the weight.
 * y    device pointer, [R, C], element `dtype`; written, rounded to nearest
 *      even.  Must not overlap x or g.
 * eps  finite, >= 0: added to the mean square before the square root.
 * Sizes, alignment, checks, ownership and asynchrony as for row_softmax.
 */
fa_status rmsnorm_silu(const void* x, const void* g, void* y, int64_t R, int64_t C, float eps, int dtype,
                       void* stream);

#ifdef __cplusplus
}
#endif

#endif /* ROWWISE_MI355X_H */
