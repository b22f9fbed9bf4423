/*
 * rowwise_oracle.c -- plain float64 CPU oracle for the two row-wise kernels:
 * the row-wise softmax and the fused RMSNorm + SiLU.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing on the product path may call, link or
 * load this file: only the tests, the smoke check and the benchmark's
 * cpu_baseline leg use it.  It shares no code, header, table or constant with
 * the HIP library.
 *
 * Row-wise softmax (the tutorial's row softmax kernel with max and sum
 * reductions kept in registers: pro.edgex.exchange summary, paragraph on the
 * fused epilogue and the row-wise softmax; datastack.it, "softmax row-wise
 * basata su reduction nei registri"), for each row x of length C:
 *     m = max_j x_j,  e_j = exp(x_j - m),  y_j = e_j / sum_j e_j
 *
 * Fused RMSNorm + SiLU (the production kernel of the pages' first summary:
 * RMSNorm followed by the SiLU activation in one kernel).  The pages give no
 * formula; the reading taken is the usual one, per row x of length C with a
 * weight g of length C:
 *     r   = 1 / sqrt(mean_j x_j^2 + eps)
 *     z_j = x_j * r * g_j
 *     y_j = silu(z_j) = z_j / (1 + exp(-z_j))
 *
 * Inputs are fp16 or bf16 bit patterns decoded exactly to double; all
 * arithmetic is double, in the order written, one row at a time.
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

/* Softmax of rows rows[0..nrows-1] of x [R, C] into y [nrows, C] doubles. */
int rowwise_oracle_softmax(const uint16_t* x, int dtype, int64_t R, int64_t C, const int64_t* rows,
                           int64_t nrows, double* y) {
    if ((dtype != 0 && dtype != 1) || R < 1 || C < 1) return -1;
    double (*dec)(uint16_t) = dtype == 0 ? decode_f16 : decode_bf16;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        if (i < 0 || i >= R) return -1;
        const uint16_t* xr = x + i * C;
        double* yr = y + r * C;
        double m = -INFINITY;
        for (int64_t j = 0; j < C; ++j)
            if (dec(xr[j]) > m) m = dec(xr[j]);
        double s = 0.0;
        for (int64_t j = 0; j < C; ++j) {
            yr[j] = exp(dec(xr[j]) - m);
            s += yr[j];
        }
        for (int64_t j = 0; j < C; ++j) yr[j] /= s;
    }
    return 0;
}

/* silu(z) = z * sigmoid(z) */
double rowwise_oracle_silu(double z) {
    return z / (1.0 + exp(-z));
}

/* RMSNorm + SiLU of rows rows[0..nrows-1] of x [R, C], weight g [C], into
 * y [nrows, C] doubles; z [nrows, C] receives the normalised, weighted
 * values before the activation when not NULL. */
int rowwise_oracle_rmsnorm_silu(const uint16_t* x, const uint16_t* g, int dtype, int64_t R, int64_t C,
                                double eps, const int64_t* rows, int64_t nrows, double* z, double* y) {
    if ((dtype != 0 && dtype != 1) || R < 1 || C < 1) return -1;
    double (*dec)(uint16_t) = dtype == 0 ? decode_f16 : decode_bf16;
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        if (i < 0 || i >= R) return -1;
        const uint16_t* xr = x + i * C;
        double ss = 0.0;
        for (int64_t j = 0; j < C; ++j) ss += dec(xr[j]) * dec(xr[j]);
        const double rs = 1.0 / sqrt(ss / (double)C + eps);
        for (int64_t j = 0; j < C; ++j) {
            const double zj = dec(xr[j]) * rs * dec(g[j]);
            if (z) z[r * C + j] = zj;
            y[r * C + j] = rowwise_oracle_silu(zj);
        }
    }
    return 0;
}
