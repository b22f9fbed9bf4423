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

#include <stddef.h>
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
    FA_ERR_LAUNCH = 3,       /* the HIP runtime refused the kernel launch (or a HIP query failed) */
    FA_ERR_SCRATCH_TOO_SMALL = 4  /* fa_fwd_split_noalloc: partials larger than FA_SPLIT_SCRATCH_BYTES */
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

/*
 * Split over the keys, for calls with few query blocks and many keys
 * (decode-shaped: small Sq, long Sk), where one work-group per (batch, head,
 * 128-query block) would leave most of the GPU idle.  The pages' online
 * softmax carries a running result across key tiles and rescales it to each
 * new maximum; here the keys of a row are cut into ranges, each range's
 * partial result (O normalised over the range, and its lse) is computed by
 * its own work-groups, and the partials are combined by the same rescaling
 * to a common maximum:
 *
 *     lse = M + ln sum_g exp(lse_g - M),   M = max_g lse_g
 *     O   = sum_g exp(lse_g - lse) O_g
 *
 * The result is the one fa_fwd computes, up to rounding.
 */

/*
 * Number of key ranges fa_fwd_split uses for this shape: n_split ranges of
 * equal length (a multiple of 64 keys, so possibly fewer ranges than asked),
 * or, for n_split = 0, a count chosen from the shape (enough ranges for about
 * 2048 work-groups, each range at least 256 keys).  0 on invalid sizes.
 */
int64_t fa_fwd_split_count(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t n_split);

/*
 * Bytes of device workspace fa_fwd_split needs for these arguments:
 * count * B*H*Sq * (D + 1) * 4 (fp32 partial O and lse per range).
 * 0 on invalid sizes.
 */
size_t fa_fwd_split_workspace_size(int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                                   int64_t n_split);

/*
 * fa_fwd_split -- enqueue the attention forward pass split over the keys:
 * the partial-result kernel, then the merge (fa_lse_merge's kernel), both on
 * `stream`.  Arguments as for fa_fwd, plus:
 *
 * n_split    ranges requested (>= 1), or 0 to let the library choose; see
 *            fa_fwd_split_count.
 * workspace  device pointer, 16-byte aligned, at least
 *            fa_fwd_split_workspace_size(B, H, Sq, Sk, D, n_split) bytes,
 *            owned by the caller and overlapping no other argument.  Once
 *            the stream has run the call, it holds the partials that were
 *            merged: O parts as fp32 [count][B*H*Sq][D] from the start, then
 *            lse parts as fp32 [count][B*H*Sq] (a row that sees no key of a
 *            range has O part 0 and lse part -inf).
 * workspace_bytes  its size; a smaller size than needed is FA_ERR_INVALID_ARG.
 *
 * Errors, ownership and asynchrony as for fa_fwd; in addition
 * B*H*ceil(Sq/128)*count must be below 2^31.  The library allocates nothing.
 */
fa_status fa_fwd_split(const void* q, const void* k, const void* v, void* o, float* lse,
                       int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                       float scale, int causal, int dtype, int64_t n_split,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * Size of the fixed device buffer of fa_fwd_split_noalloc: 32 MiB, held by
 * every device the library runs on from the first such call until the
 * process ends.
 */
#define FA_SPLIT_SCRATCH_BYTES (32u * 1024u * 1024u)

/*
 * fa_fwd_split_noalloc -- fa_fwd_split with its partial results in a fixed
 * device buffer inside the library instead of a caller workspace, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid allocation).  It calls no
 * allocating routine.
 *
 * Arguments, checks, results and asynchrony as for fa_fwd_split, without
 * the workspace.  The partials must fit the buffer:
 * fa_fwd_split_workspace_size(B, H, Sq, Sk, D, n_split) <= FA_SPLIT_SCRATCH_BYTES,
 * else FA_ERR_SCRATCH_TOO_SMALL and nothing is launched (a smaller n_split
 * needs less).  The buffer's device address is looked up on the first call
 * made with a device current (hipGetDevice), so `stream` must belong to the
 * current device.  Every call on a device shares that device's buffer, which
 * keeps the last call's partials: calls that overlap on one device (other
 * streams, or other threads, without ordering between them) race and give
 * wrong results.  Nothing in the buffer needs to start at zero: each call
 * writes every partial it reads.
 */
fa_status fa_fwd_split_noalloc(const void* q, const void* k, const void* v, void* o, float* lse,
                               int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                               float scale, int causal, int dtype, int64_t n_split, void* stream);

/*
 * fa_lse_merge -- enqueue the log-sum-exp merge of partial attention results
 * over disjoint key ranges (formula above), for rows computed anywhere (for
 * example key ranges held by different devices).
 *
 * o_parts    device pointer, fp32 [n_part][rows][D], 16-byte aligned: each
 *            part's O, normalised over its keys (0 for an empty part).
 * lse_parts  device pointer, fp32 [n_part][rows]: each part's lse (-inf for
 *            an empty part).
 * n_part >= 1, rows >= 1, D = 64 or 128.
 * o          device pointer, [rows][D] of `dtype`, 16-byte aligned; written,
 *            rounded to nearest even.
 * lse        device pointer, fp32 [rows]; written.  A row whose parts are
 *            all empty gets lse -inf and O 0.
 * The outputs must not overlap the inputs.  Checks, errors and asynchrony
 * as for fa_fwd; NaN parts propagate.
 */
fa_status fa_lse_merge(const float* o_parts, const float* lse_parts, int64_t n_part, int64_t rows,
                       int64_t D, void* o, float* lse, int dtype, void* stream);

/* Static, never-NULL description of a status code (unknown codes included). */
const char* fa_status_string(int status);

#ifdef __cplusplus
}
#endif

#endif /* FA_MI355X_H */
