/*
 * fa_oracle.c -- plain float64 CPU oracle for the fused attention forward pass.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (the plain definition; the fused kernel reaches the same
 * result up to rounding):
 *
 *   For every (b, h) and query row i:
 *     s_j  = scale * sum_d q[i][d] * k[j][d]          (all Sk keys, explicit)
 *     s_j  = -inf  if causal and j > i                 (top-left alignment)
 *     m    = max_j s_j
 *     p_j  = exp(s_j - m)
 *     l    = sum_j p_j
 *     o[i][d] = (sum_j p_j * v[j][d]) / l
 *     lse[i]  = m + ln(l)
 *
 * Source: "TileLang ... FlashAttention" write-ups (MarkTechPost tutorial as
 * summarised on pro.edgex.exchange, paragraph on the fused FlashAttention
 * forward kernel): the kernel computes softmax attention over Q, K, V tiles
 * with running maxima, normalising sums and rescale factors, causal and
 * non-causal, and is validated against PyTorch's scaled-dot-product attention.
 * The pages write no formula; the formula above is the scaled-dot-product
 * attention definition those checks compare against.  The mask is top-left
 * aligned (key j hidden from query i when j > i, for any Sq and Sk), the lse
 * is the natural log of the normalising sum of the scaled logits, and the
 * layout is contiguous [B, H, S, D] with D fastest.
 *
 * Two more routines serve a split over the keys: fa_oracle_rows_range (the
 * same rows over a key range) and fa_oracle_merge (the log-sum-exp merge of
 * partial results; see there).
 *
 * Inputs are fp16 or bf16 bit patterns (uint16); they are decoded exactly to
 * double.  All arithmetic is double, in the order written above, one row at
 * a time, with no tiling or online rescaling.  Rows are independent, so a
 * caller may evaluate any subset of rows (row = (b*H + h)*Sq + i).
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ---- exact decoding of the storage formats ------------------------------ */

/* IEEE binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits. */
static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);               /* subnormal: f * 2^-14 * 2^-10 */
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);  /* (1.f) * 2^(e-15) */
    return sign ? -v : v;
}

/* bfloat16: the upper 16 bits of an IEEE binary32. */
static double decode_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);              /* subnormal: f * 2^-126 * 2^-7 */
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x80), e - 134);  /* (1.f) * 2^(e-127) */
    return sign ? -v : v;
}

static double g_tab[2][65536];
static int g_ready = 0;

/* Fill the decode tables.  Call once before any other entry point (the
 * Python wrapper does so when it loads the library). */
void fa_oracle_init(void) {
    if (g_ready) return;
    for (int i = 0; i < 65536; ++i) {
        g_tab[0][i] = decode_f16((uint16_t)i);
        g_tab[1][i] = decode_bf16((uint16_t)i);
    }
    g_ready = 1;
}

/* Decode n bit patterns to double (dtype 0 = fp16, 1 = bf16). */
void fa_oracle_decode(const uint16_t* bits, int64_t n, int dtype, double* out) {
    for (int64_t i = 0; i < n; ++i) out[i] = g_tab[dtype][bits[i]];
}

/*
 * Evaluate rows rows[0..nrows-1] (flat row index (b*H + h)*Sq + i) over the
 * keys k_begin <= j < k_end only (0 <= k_begin < k_end <= Sk); the causal mask
 * uses the global key index j.  This is the same row computation with the
 * other keys left out, as when the keys of a row are split into ranges.  A
 * row that sees no key of the range (causal, i < k_begin) has an empty
 * softmax: its lse is -inf and its o is 0, which gives it zero weight in
 * fa_oracle_merge.
 * q: [B,H,Sq,D]; k, v: [B,H,Sk,D] bit patterns.  o: [nrows, D] doubles,
 * lse: [nrows] doubles.  Returns 0, or -1 on bad arguments / no memory.
 */
int fa_oracle_rows_range(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                         int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                         double scale, int causal, int64_t k_begin, int64_t k_end,
                         const int64_t* rows, int64_t nrows, double* o, double* lse) {
    if (!g_ready || (dtype != 0 && dtype != 1) || B < 1 || H < 1 || Sq < 1 || Sk < 1 || D < 1)
        return -1;
    if (k_begin < 0 || k_end > Sk || k_begin >= k_end)
        return -1;
    const double* tab = g_tab[dtype];
    double* qd = (double*)malloc(sizeof(double) * (size_t)D);
    double* s = (double*)malloc(sizeof(double) * (size_t)Sk);
    double* acc = (double*)malloc(sizeof(double) * (size_t)D);
    if (!qd || !s || !acc) {
        free(qd); free(s); free(acc);
        return -1;
    }
    for (int64_t r = 0; r < nrows; ++r) {
        int64_t row = rows[r];
        if (row < 0 || row >= B * H * Sq) { free(qd); free(s); free(acc); return -1; }
        int64_t bh = row / Sq;
        int64_t i = row % Sq;
        const uint16_t* qrow = q + row * D;
        const uint16_t* kh = k + bh * Sk * D;
        const uint16_t* vh = v + bh * Sk * D;

        for (int64_t d = 0; d < D; ++d) qd[d] = tab[qrow[d]];

        /* scores, explicit, with the mask applied after scaling */
        for (int64_t j = k_begin; j < k_end; ++j) {
            if (causal && j > i) {
                s[j] = -INFINITY;
                continue;
            }
            double dot = 0.0;
            for (int64_t d = 0; d < D; ++d) dot += qd[d] * tab[kh[j * D + d]];
            s[j] = scale * dot;
        }

        /* softmax */
        double m = -INFINITY;
        for (int64_t j = k_begin; j < k_end; ++j)
            if (s[j] > m) m = s[j];
        if (m == -INFINITY) {       /* no visible key in the range: empty softmax */
            for (int64_t d = 0; d < D; ++d) o[r * D + d] = 0.0;
            lse[r] = -INFINITY;
            continue;
        }
        double l = 0.0;
        for (int64_t j = k_begin; j < k_end; ++j) {
            s[j] = exp(s[j] - m);   /* s now holds p_j; exp(-inf) = 0 */
            l += s[j];
        }

        /* output */
        for (int64_t d = 0; d < D; ++d) acc[d] = 0.0;
        for (int64_t j = k_begin; j < k_end; ++j) {
            double p = s[j];
            for (int64_t d = 0; d < D; ++d) acc[d] += p * tab[vh[j * D + d]];
        }
        for (int64_t d = 0; d < D; ++d) o[r * D + d] = acc[d] / l;
        lse[r] = m + log(l);
    }
    free(qd); free(s); free(acc);
    return 0;
}

/* All Sk keys: the definition in the header comment. */
int fa_oracle_rows(const uint16_t* q, const uint16_t* k, const uint16_t* v, int dtype,
                   int64_t B, int64_t H, int64_t Sq, int64_t Sk, int64_t D,
                   double scale, int causal,
                   const int64_t* rows, int64_t nrows, double* o, double* lse) {
    return fa_oracle_rows_range(q, k, v, dtype, B, H, Sq, Sk, D, scale, causal, 0, Sk,
                                rows, nrows, o, lse);
}

/*
 * Merge of partial results over disjoint key ranges that together cover a
 * row's keys.  The pages' online softmax combines the running result of the
 * keys seen so far with a new tile's by rescaling both to a common maximum;
 * two finished partial results combine the same way.  With part g holding
 * o_g (normalised over its keys) and lse_g = m_g + ln l_g, for each row:
 *   M   = max_g lse_g
 *   lse = M + ln( sum_g exp(lse_g - M) )
 *   o   = sum_g exp(lse_g - lse) * o_g
 * Parts with lse_g = -inf (empty ranges) get zero weight; a row whose parts
 * are all empty gets lse = -inf and o = 0.
 * o_parts: [n_part][nrows][D], lse_parts: [n_part][nrows]; o: [nrows][D],
 * lse: [nrows].  Returns 0, or -1 on bad arguments.
 */
int fa_oracle_merge(int64_t n_part, int64_t nrows, int64_t D, const double* o_parts,
                    const double* lse_parts, double* o, double* lse) {
    if (n_part < 1 || nrows < 0 || D < 1) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        double M = -INFINITY;
        for (int64_t g = 0; g < n_part; ++g)
            if (lse_parts[g * nrows + r] > M) M = lse_parts[g * nrows + r];
        for (int64_t d = 0; d < D; ++d) o[r * D + d] = 0.0;
        if (M == -INFINITY) {
            lse[r] = -INFINITY;
            continue;
        }
        double sum = 0.0;
        for (int64_t g = 0; g < n_part; ++g) sum += exp(lse_parts[g * nrows + r] - M);
        lse[r] = M + log(sum);
        for (int64_t g = 0; g < n_part; ++g) {
            double w = exp(lse_parts[g * nrows + r] - lse[r]);
            for (int64_t d = 0; d < D; ++d) o[r * D + d] += w * o_parts[(g * nrows + r) * D + d];
        }
    }
    return 0;
}
