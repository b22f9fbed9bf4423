/*
 * fa.h -- C ABI of the MI355X (gfx950) fused attention forward library.
 *
 * The operation is the fused FlashAttention forward pass described on the
 * TileLang tutorial pages (pro.edgex.exchange summary, paragraph on the fused
 * FlashAttention forward kernel; comrad404.com, section "Как устроен
 * туториал", FlashAttention paragraph; datastack.it, section "Cosa copre il
 * tutorial"): for every (batch, head) it computes
 *
 *     O   = softmax(scale * Q K^T + M) V        M = causal mask or 0
 *     lse = log(sum_j exp(scale * q_i . k_j))   over the keys row i sees
 *
 * tile by tile with an online softmax (running row maximum, running
 * normalising sum, rescale factors), so the score matrix never reaches
 * device memory.  The pages validate causal and non-causal attention against
 * PyTorch's scaled-dot-product attention; the layout and mask follow that
 * routine's conventions.
 *
 * Nothing here includes HIP headers: pointers are plain device addresses and
 * the stream is a hipStream_t passed as void*.
 */
#ifndef FA_MI355X_H
#define FA_MI355X_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* Element type of q, k, v and o. */
typedef enum {
    FA_F16 = 0,  /* IEEE binary16 */
    FA_BF16 = 1  /* bfloat16 */
} fa_dtype;

typedef enum {
    FA_OK = 0,
    FA_ERR_INVALID_ARG = 1,  /* null or misaligned pointer, bad size, overlap, non-finite scale */
    FA_ERR_UNSUPPORTED = 2,  /* head dimension or dtype this build does not provide */
    FA_ERR_LAUNCH = 3        /* the HIP runtime refused the kernel launch */
} fa_status;

/*
 * fa_fwd -- enqueue one fused attention forward pass on `stream`.
 *
 * q    device pointer, [B, H, Sq, D] contiguous (D fastest), element `dtype`.
 * k, v device pointers, [B, H, Sk, D] contiguous, element `dtype`.
 * o    device pointer, [B, H, Sq, D] contiguous, element `dtype`; written.
 * lse  device pointer, [B, H, Sq] contiguous float32; written with the natural
 *      log of the softmax normaliser of each row, in units of the scaled logits
 *      (lse_i = max_j s_ij + ln sum_j exp(s_ij - max_j s_ij), s = scale*q.k).
 * B, H, Sq, Sk  >= 1.  D must be 64 or 128.
 * scale  finite; multiplies q.k before masking and softmax (any sign).
 * causal 0: every row sees all Sk keys.  Non-zero: top-left alignment, row i
 *        sees keys 0 .. min(i, Sk-1) (key j is hidden when j > i), for any
 *        Sq and Sk.  Every row therefore sees at least key 0.
 * dtype  an fa_dtype value.
 * stream a hipStream_t (NULL = the null stream).
 *
 * Alignment: q, k, v and o must be 16-byte aligned, lse 4-byte aligned.
 * Ownership: the caller owns every buffer.  The library allocates nothing,
 * keeps no state between calls and does not retain pointers.  q, k, v are
 * read only; o and lse must not overlap q, k, v or each other.
 *
 * The call checks its arguments on the host (no device access) and returns
 * an error code without launching anything if one is wrong.  On FA_OK the
 * kernel has been enqueued and the call returns without synchronising:
 * results are valid once the caller synchronises `stream`.  Faults inside
 * the kernel surface at that synchronisation.  Input values are not
 * inspected: NaN or Inf inputs propagate to the outputs of the rows they
 * reach.  Repeated calls on identical inputs give bit-identical outputs.
 *
 * Limits: Sq*D and Sk*D must be below 2^31, and B*H*ceil(Sq/128) below 2^31.
 */
fa_status fa_fwd(const void* q, const void* k, const void* v, void* o, float* lse,
                 int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                 float scale, int causal, int dtype, void* stream);

/* Static, never-NULL description of a status code (unknown codes included). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
