/*
 * gemm_oracle.c -- plain float64 CPU oracle for the GEMM with a fused bias +
 * GELU epilogue.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * What it computes (the TileLang tutorial's fused-epilogue GEMM: the bias
 * addition and the GELU activation applied to the accumulator before the
 * output is written -- MarkTechPost tutorial as summarised on
 * pro.edgex.exchange, paragraph on the fused GEMM epilogue; datastack.it,
 * section "Cosa copre il tutorial", "GEMM + bias + GELU in un solo kernel"):
 *
 *   x[m][n] = sum_k a[m][k] * w[n][k] + bias[n]
 *   c[m][n] = gelu(x[m][n]) = x * Phi(x) = 0.5 * x * (1 + erf(x / sqrt(2)))
 *
 * The pages fix neither the layout nor the GELU form; this is the eager
 * PyTorch expression the tutorial compares against, gelu(a @ w.T + bias):
 * a is [M, K], w is [N, K] (the weight layout of a linear layer), bias [N],
 * c [M, N], all row-major, and GELU is the exact (erf) form, PyTorch's
 * default.  Inputs are fp16 or bf16 bit patterns decoded exactly to double;
 * all arithmetic is double, one output element at a time, k in order.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>

static double decode_f16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 10) & 0x1F;
    int f = h & 0x3FF;
    double v;
    if (e == 0)
        v = ldexp((double)f, -24);
    else if (e == 31)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x400), e - 25);
    return sign ? -v : v;
}

static double decode_bf16(uint16_t h) {
    int sign = (h >> 15) & 1;
    int e = (h >> 7) & 0xFF;
    int f = h & 0x7F;
    double v;
    if (e == 0)
        v = ldexp((double)f, -133);
    else if (e == 255)
        v = f ? NAN : INFINITY;
    else
        v = ldexp((double)(f | 0x80), e - 134);
    return sign ? -v : v;
}

/* gelu(x) = x * Phi(x), Phi the standard normal distribution function. */
double gemm_oracle_gelu(double x) {
    return 0.5 * x * (1.0 + erf(x / sqrt(2.0)));
}

/*
 * Output rows rows[0..nrows-1] of c (all N columns of each).  a: [M,K],
 * w: [N,K], bias: [N] (NULL: no bias) as bit patterns of `dtype` (0 fp16,
 * 1 bf16).  pre: [nrows, N] doubles receiving x (may be NULL); c: [nrows, N]
 * doubles receiving gelu(x).  Returns 0, or -1 on bad arguments or memory.
 */
int gemm_oracle_rows(const uint16_t* a, const uint16_t* w, const uint16_t* bias, int dtype,
                     int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows,
                     double* pre, double* c) {
    if ((dtype != 0 && dtype != 1) || M < 1 || N < 1 || K < 1) return -1;
    double (*dec)(uint16_t) = dtype == 0 ? decode_f16 : decode_bf16;
    double* ar = (double*)malloc(sizeof(double) * (size_t)K);
    if (!ar) return -1;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t m = rows[r];
        if (m < 0 || m >= M) { free(ar); return -1; }
        for (int64_t k = 0; k < K; ++k) ar[k] = dec(a[m * K + k]);
        for (int64_t n = 0; n < N; ++n) {
            double x = 0.0;
            for (int64_t k = 0; k < K; ++k) x += ar[k] * dec(w[n * K + k]);
            if (bias) x += dec(bias[n]);
            if (pre) pre[r * N + n] = x;
            c[r * N + n] = gemm_oracle_gelu(x);
        }
    }
    free(ar);
    return 0;
}
