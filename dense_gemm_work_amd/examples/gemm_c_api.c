/*
 * gemm_c_api.c -- the C ABI used from plain C: device buffers from the HIP
 * runtime, one heuristic call (3 x 2 tiles of 5 k-iterations, ragged in M and
 * N: the rule stays data-parallel), one Stream-K call with 7 units and a fused
 * epilogue through gemm_ex, one heuristic call with the tile left to the
 * library (GEMM_TILE_AUTO), and a host check of each.
 *
 * Build (done by dense_gemm_work_amd/build.py):
 *   hipcc -x c ... gemm_c_api.c -L<pkg> -ldgw_gemm -o gemm_c_api
 * Run: ./gemm_c_api  -> prints the largest relative error of each call and
 * exits 0 when all are within their bounds (1e-4 of sum|a||b| for the products).
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "../../include/gemm.h"

/* bf16 by truncation of an fp32 value that is exactly representable: the
 * inputs below are small integers divided by 8, so nothing is lost. */
static uint16_t to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    return (uint16_t)(u >> 16);
}

#define CHECK_HIP(x)                                                       \
    do {                                                                   \
        hipError_t e_ = (x);                                               \
        if (e_ != hipSuccess) {                                            \
            fprintf(stderr, "%s: %s\n", #x, hipGetErrorString(e_));       \
            return 2;                                                      \
        }                                                                  \
    } while (0)

int main(void) {
    const int64_t M = 300, N = 200, K = 320;
    float *a = malloc(sizeof(float) * M * K), *b = malloc(sizeof(float) * K * N);
    uint16_t *ah = malloc(2 * M * K), *bh = malloc(2 * K * N);
    float *c = malloc(sizeof(float) * M * N), *bias = malloc(sizeof(float) * N);
    double *ref = malloc(sizeof(double) * M * N), *mag = malloc(sizeof(double) * M * N);
    if (!a || !b || !ah || !bh || !c || !bias || !ref || !mag) return 2;
    for (int64_t i = 0; i < M * K; ++i) a[i] = (float)((i * 7 + 3) % 17 - 8) / 8.0f;
    for (int64_t i = 0; i < K * N; ++i) b[i] = (float)((i * 5 + 1) % 13 - 6) / 8.0f;
    for (int64_t j = 0; j < N; ++j) bias[j] = (float)(j % 5) - 2.0f;
    for (int64_t i = 0; i < M * K; ++i) ah[i] = to_bf16(a[i]);
    for (int64_t i = 0; i < K * N; ++i) bh[i] = to_bf16(b[i]);
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            double s = 0, m = 0;
            for (int64_t k = 0; k < K; ++k) {
                s += (double)a[i * K + k] * b[k * N + j];
                m += fabs((double)a[i * K + k] * b[k * N + j]);
            }
            ref[i * N + j] = s;
            mag[i * N + j] = m;
        }

    void *dA, *dB, *dBias;
    float *dC;
    CHECK_HIP(hipMalloc(&dA, 2 * M * K));
    CHECK_HIP(hipMalloc(&dB, 2 * K * N));
    CHECK_HIP(hipMalloc((void **)&dC, 4 * M * N));
    CHECK_HIP(hipMalloc(&dBias, 4 * N));
    CHECK_HIP(hipMemcpy(dA, ah, 2 * M * K, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dB, bh, 2 * K * N, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dBias, bias, 4 * N, hipMemcpyHostToDevice));

    /* 1: C = A.B, heuristic decomposition */
    gemm_plan_t plan;
    if (gemm_plan(M, N, K, GEMM_B_KN | GEMM_BF16, GEMM_HEURISTIC, 0, gemm_num_cus(), &plan) != GEMM_OK) {
        fprintf(stderr, "gemm_plan: %s\n", gemm_last_error());
        return 1;
    }
    if (gemm(dA, dB, dC, M, N, K, GEMM_B_KN | GEMM_BF16, GEMM_HEURISTIC, 0) != GEMM_OK) {
        fprintf(stderr, "gemm: %s\n", gemm_last_error());
        return 1;
    }
    if (gemm_sync_status(NULL) != GEMM_OK) {
        fprintf(stderr, "gemm_sync_status: %s\n", gemm_last_error());
        return 1;
    }
    CHECK_HIP(hipMemcpy(c, dC, 4 * M * N, hipMemcpyDeviceToHost));
    double worst = 0;
    for (int64_t i = 0; i < M * N; ++i) {
        const double r = fabs(c[i] - ref[i]) / (1e-4 * mag[i] + 1e-30);
        if (r > worst) worst = r;
    }
    printf("gemm: decision %d, %lld tiles, worst |err| / (1e-4 sum|a||b|) = %.3e\n", plan.decision,
           (long long)plan.tiles, worst);
    int ok = worst <= 1.0;

    /* 2: C = relu(2 A.B - C + bias) through gemm_ex (C holds the product from call 1) */
    gemm_args_t args;
    memset(&args, 0, sizeof args);
    args.A = dA;
    args.B = dB;
    args.C = dC;
    args.M = M;
    args.N = N;
    args.K = K;
    args.layout = GEMM_B_KN | GEMM_BF16;
    args.mode = GEMM_STREAMK;
    args.splits = 7;
    args.epilogue = GEMM_EPI_ALPHA_BETA | GEMM_EPI_BIAS | GEMM_EPI_RELU;
    args.alpha = 2.0f;
    args.beta = -1.0f;
    args.bias = (const float *)dBias;
    if (gemm_ex(&args) != GEMM_OK || gemm_sync_status(NULL) != GEMM_OK) {
        fprintf(stderr, "gemm_ex: %s\n", gemm_last_error());
        return 1;
    }
    float *c2 = malloc(sizeof(float) * M * N);
    if (!c2) return 2;
    CHECK_HIP(hipMemcpy(c2, dC, 4 * M * N, hipMemcpyDeviceToHost));
    double worst2 = 0;
    for (int64_t i = 0; i < M; ++i)
        for (int64_t j = 0; j < N; ++j) {
            const int64_t x = i * N + j;
            double y = 2.0 * ref[x] - c[x] + bias[j];
            y = y > 0 ? y : 0;
            const double bound = 2e-4 * mag[x] + 1e-6 * (fabs(2.0 * ref[x]) + fabs(c[x]) + fabs(bias[j])) + 1e-30;
            const double r = fabs(c2[x] - y) / bound;
            if (r > worst2) worst2 = r;
        }
    printf("gemm_ex epilogue: worst |err| / bound = %.3e\n", worst2);
    ok = ok && worst2 <= 1.0;

    /* 3: C = A.B, the library picking the tile: 6 tiles of 128 x 128 would fill
     * few CUs, so it takes 64 x 128 */
    gemm_plan_t plan3;
    const uint32_t mode3 = GEMM_HEURISTIC | GEMM_TILE_AUTO;
    if (gemm_plan(M, N, K, GEMM_B_KN | GEMM_BF16, mode3, 0, gemm_num_cus(), &plan3) != GEMM_OK ||
        gemm(dA, dB, dC, M, N, K, GEMM_B_KN | GEMM_BF16, mode3, 0) != GEMM_OK || gemm_sync_status(NULL) != GEMM_OK) {
        fprintf(stderr, "gemm with GEMM_TILE_AUTO: %s\n", gemm_last_error());
        return 1;
    }
    CHECK_HIP(hipMemcpy(c2, dC, 4 * M * N, hipMemcpyDeviceToHost));
    double worst3 = 0;
    for (int64_t i = 0; i < M * N; ++i) {
        const double r = fabs(c2[i] - ref[i]) / (1e-4 * mag[i] + 1e-30);
        if (r > worst3) worst3 = r;
    }
    printf("gemm GEMM_TILE_AUTO: %d x %d tiles, worst |err| / (1e-4 sum|a||b|) = %.3e\n", plan3.bm, plan3.bn, worst3);
    ok = ok && worst3 <= 1.0;

    hipFree(dA);
    hipFree(dB);
    hipFree(dC);
    hipFree(dBias);
    gemm_release();
    free(a), free(b), free(ah), free(bh), free(c), free(c2), free(bias), free(ref), free(mag);
    printf("%s\n", ok ? "ok" : "FAILED");
    return ok ? 0 : 1;
}
