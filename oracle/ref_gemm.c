/*
 * ref_gemm.c -- plain fp64 reference GEMM over 16-bit operand bit patterns.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the value oracle that the HIP path
 * is checked against.  Only tests/, the smoke check and the benchmark's CPU
 * baseline leg may load it; the library itself never does.  It shares no code
 * with the HIP path.
 *
 * What it computes (Split-K/Stream-K book chapter, "Case 3" correctness check
 * and "The boring rule": validate against an fp64 reference with a K-scaled
 * tolerance; Metal split-K note, "Contract and numerical coverage": fp64 dot
 * products over the actual dtype-rounded inputs):
 *
 *     C[i][j] = sum_k a[i][k] * b[k][j]          (fp64, k ascending)
 *     S[i][j] = sum_k |a[i][k]| * |b[k][j]|      (fp64, k ascending)
 *
 * with b[k][j] = B[k*N + j] when B is stored [K,N] ("kn") and
 * b[k][j] = B[j*K + k] when B is stored [N,K] ("nk", i.e. C = A.B^T).
 *
 * Operands arrive as raw bf16 or fp16 bit patterns and are decoded exactly to
 * fp64 from the format definitions (bfloat16 = the upper half of an IEEE
 * binary32; fp16 = IEEE binary16).  Every product of two such values is exact
 * in fp64, so the only rounding is the fp64 accumulation.
 *
 * Loop order i-k-j accumulates every C[i][j] in ascending k; rows are
 * independent and are spread over OpenMP threads.  There is no blocking and
 * no reordering of any element's sum.
 *
 * Pins (tests/test_oracle_gemm.py): format decoding of known bit patterns,
 * exact integer results, closed forms (all-ones, alternating signs, zero row),
 * brute-force rational sums on tiny inputs, numpy float64 matmul, layout
 * transposition, and planted-mistake builds (ORACLE_MUTATION) that must fail.
 */
#include <math.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

#ifdef _OPENMP
#include <omp.h>
#endif

#ifndef ORACLE_MUTATION
#define ORACLE_MUTATION 0
#endif

/* bfloat16: the upper 16 bits of an IEEE-754 binary32. */
double oracle_bf16_to_f64(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, sizeof f);
    return (double)f;
}

/* IEEE-754 binary16: 1 sign bit, 5 exponent bits (bias 15), 10 fraction bits. */
double oracle_fp16_to_f64(uint16_t h) {
    int sign = (h >> 15) & 1;
    int ex = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (ex == 0) {
        v = ldexp((double)frac, -24);                 /* subnormal: frac * 2^-24 */
    } else if (ex == 0x1f) {
        v = frac ? NAN : INFINITY;
    } else {
#if ORACLE_MUTATION == 4
        v = ldexp((double)(0x400 | frac), ex - 24);   /* planted: wrong exponent bias */
#else
        v = ldexp((double)(0x400 | frac), ex - 25);   /* (1.frac) * 2^(ex-15) */
#endif
    }
    return sign ? -v : v;
}

static double decode(uint16_t h, int dtype) {
    return dtype == 1 ? oracle_fp16_to_f64(h) : oracle_bf16_to_f64(h);
}

int oracle_num_threads(void) {
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/*
 * Reference GEMM on a subset of rows.
 *   A: [M,K] row-major bit patterns; B: [K,N] (b_layout 0) or [N,K] (b_layout 1).
 *   dtype: 0 = bf16, 1 = fp16.
 *   rows[r] (r < nrows) selects the rows of C to compute; C and S receive
 *   nrows x N doubles, row r of the output being row rows[r] of the product.
 *   S may be NULL.
 * Returns 0, or -1 on a bad argument.
 */
int oracle_gemm_rows(const uint16_t *A, const uint16_t *B, int64_t M, int64_t N, int64_t K,
                     int b_layout, int dtype, const int64_t *rows, int64_t nrows,
                     double *C, double *S) {
    if (M < 0 || N < 0 || K < 0 || nrows < 0 || (b_layout != 0 && b_layout != 1) ||
        (dtype != 0 && dtype != 1))
        return -1;
    for (int64_t r = 0; r < nrows; ++r)
        if (rows[r] < 0 || rows[r] >= M) return -1;
    if (nrows == 0 || N == 0) return 0;

    /* Decode B once into a [K][N] array of b[k][j]. */
    double *bd = (double *)malloc((size_t)(K > 0 ? K : 1) * (size_t)N * sizeof(double));
    if (!bd) return -1;
#pragma omp parallel for schedule(static)
    for (int64_t k = 0; k < K; ++k) {
        for (int64_t j = 0; j < N; ++j) {
#if ORACLE_MUTATION == 2
            /* planted: reads the stored matrix with the other layout's index */
            uint16_t h = b_layout == 0 ? B[j * K + k] : B[k * N + j];
#else
            uint16_t h = b_layout == 0 ? B[k * N + j] : B[j * K + k];
#endif
            bd[k * N + j] = decode(h, dtype);
        }
    }

#pragma omp parallel for schedule(dynamic, 1)
    for (int64_t r = 0; r < nrows; ++r) {
        const int64_t i = rows[r];
        double *c = C + r * N;
        double *s = S ? S + r * N : NULL;
        for (int64_t j = 0; j < N; ++j) c[j] = 0.0;
        if (s)
            for (int64_t j = 0; j < N; ++j) s[j] = 0.0;
#if ORACLE_MUTATION == 1
        const int64_t kend = K > 0 ? K - 1 : 0;      /* planted: drops the last k term */
#else
        const int64_t kend = K;
#endif
        for (int64_t k = 0; k < kend; ++k) {
            const double a = decode(A[i * K + k], dtype);
            const double *b = bd + k * N;
            for (int64_t j = 0; j < N; ++j) c[j] += a * b[j];
            if (s) {
                const double aa = fabs(a);
#if ORACLE_MUTATION == 3
                for (int64_t j = 0; j < N; ++j) s[j] += aa * b[j];  /* planted: |b| dropped */
#else
                for (int64_t j = 0; j < N; ++j) s[j] += aa * fabs(b[j]);
#endif
            }
        }
    }
    free(bd);
    return 0;
}
