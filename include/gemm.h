/*
 * gemm.h -- C ABI of the GEMM with a fused bias + GELU epilogue (gfx950).
 *
 * The operation is the TileLang tutorial's fused-epilogue GEMM: a tiled
 * tensor-core matrix multiplication whose bias addition and GELU activation
 * are applied to the accumulator held in registers, before the output tile
 * is written, instead of as separate passes over global memory
 * (pro.edgex.exchange summary, paragraph on the fused GEMM epilogue;
 * datastack.it, section "Cosa copre il tutorial"; comrad404.com, section on
 * fusion).  The pages compare it against eager PyTorch; the expression taken
 * is that eager one:
 *
 *     C = gelu(A W^T + bias),   gelu(x) = x * Phi(x) = x/2 * (1 + erf(x / sqrt(2)))
 *
 * (the exact, erf form of GELU, PyTorch's default; W in the [N, K] layout
 * of a linear layer's weight).
 *
 * Status codes and element types are those of fa.h.
 */
#ifndef GEMM_MI355X_H
#define GEMM_MI355X_H

#include <stdint.h>

#include "fa.h"

#ifdef __cplusplus
extern "C" {
#endif

/*
 * gemm_bias_gelu -- enqueue C = gelu(A W^T + bias) on `stream`.
 *
 * a     device pointer, [M, K] row-major (K fastest), element `dtype`,
 *       16-byte aligned.
 * w     device pointer, [N, K] row-major, element `dtype`, 16-byte aligned.
 * bias  device pointer, [N], element `dtype`, 2-byte aligned; NULL means no
 *       bias (zero).
 * c     device pointer, [M, N] row-major, element `dtype`, 16-byte aligned;
 *       written, rounded to nearest even from the fp32 result.
 * M, N, K >= 1; K must be a multiple of 8 (rows of 16-byte chunks),
 *       otherwise FA_ERR_UNSUPPORTED.  M, N, K < 2^31, 256*K < 2^32 - 16,
 *       and ceil(M/256)*ceil(N/256) < 2^31.
 * dtype FA_F16 or FA_BF16.
 * stream a hipStream_t (NULL = the null stream).
 *
 * Products are accumulated in fp32; bias and GELU are applied in fp32.
 * The caller owns every buffer; the library allocates nothing and keeps
 * no pointer.  c must not overlap a, w or bias.  Arguments are checked on
 * the host before any device access; on FA_OK the kernel is enqueued and
 * the call returns without synchronising.  NaN or Inf inputs propagate to
 * the outputs they reach.  Repeated calls give bit-identical outputs.
 */
fa_status gemm_bias_gelu(const void* a, const void* w, const void* bias, void* c,
                         int64_t M, int64_t N, int64_t K, int dtype, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* GEMM_MI355X_H */
