/*
 * c_abi_gpu.c -- test program: the library used from plain C with the HIP
 * runtime's C API for device memory (no C++, no Python, no PyTorch).  A
 * small bf16 problem (m = 37 tokens, top-3 of 9 experts, n = 70, k = 296):
 * Direct and Grouped matmul_id, compared bit for bit with each other and
 * within 2e-5 (relative to max(1, |ref|)) of a double-precision reference
 * computed here.  Exit status 0 on success; prints the worst error.
 */
#include <hip/hip_runtime_api.h>
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

#include "eidm.h"

enum { M = 37, TOPK = 3, E = 9, N = 70, K = 296 };

#define CHECK_HIP(x)                                                                  \
    do {                                                                              \
        hipError_t e_ = (x);                                                          \
        if (e_ != hipSuccess) {                                                       \
            printf("hip error %d at %s:%d\n", (int)e_, __FILE__, __LINE__);           \
            return 2;                                                                 \
        }                                                                             \
    } while (0)

static uint32_t lcg(uint64_t* st) {
    *st = *st * 6364136223846793005ull + 1442695040888963407ull;
    return (uint32_t)(*st >> 33);
}

static float bf16_to_f32(uint16_t h) {
    uint32_t u = (uint32_t)h << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

int main(void) {
    uint64_t st = 12345;
    static uint16_t w[E * N * K];
    static float x[M * K];
    static uint32_t ids[M * TOPK];
    static float yd[M * TOPK * N], yg[M * TOPK * N];
    for (int i = 0; i < E * N * K; ++i) {
        /* weights in [-1/8, 1/8): small integers over 1024, exact in bf16 */
        float v = ((int)(lcg(&st) % 256) - 128) / 1024.0f;
        uint32_t u;
        memcpy(&u, &v, 4);
        w[i] = (uint16_t)(u >> 16);
    }
    for (int i = 0; i < M * K; ++i) x[i] = ((int)(lcg(&st) % 2001) - 1000) / 997.0f;
    for (int t = 0; t < M; ++t)
        for (int s = 0; s < TOPK; ++s) ids[t * TOPK + s] = (uint32_t)((t * 5 + s * 2) % E);  /* distinct per token */

    eidm_shape sh;
    memset(&sh, 0, sizeof sh);
    sh.struct_size = sizeof sh;
    sh.weight_dtype = EIDM_DTYPE_BF16;
    sh.m = M;
    sh.n = N;
    sh.k = K;
    sh.top_k = TOPK;
    sh.n_experts = E;
    sh.expert_stride_bytes = (uint64_t)N * K * 2;
    eidm_requirements rq;
    memset(&rq, 0, sizeof rq);
    rq.struct_size = sizeof rq;
    if (eidm_query(&sh, EIDM_ROUTE_GROUPED, &rq) != EIDM_OK) {
        printf("query failed: %s\n", eidm_last_error());
        return 1;
    }
    void *dw, *dx, *dids, *dy, *dscr;
    CHECK_HIP(hipMalloc(&dw, sizeof w));
    CHECK_HIP(hipMalloc(&dx, sizeof x));
    CHECK_HIP(hipMalloc(&dids, sizeof ids));
    CHECK_HIP(hipMalloc(&dy, sizeof yd));
    CHECK_HIP(hipMalloc(&dscr, rq.scratch_bytes));
    CHECK_HIP(hipMemcpy(dw, w, sizeof w, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dx, x, sizeof x, hipMemcpyHostToDevice));
    CHECK_HIP(hipMemcpy(dids, ids, sizeof ids, hipMemcpyHostToDevice));
    int taken = 0;
    if (eidm_matmul_id(&sh, EIDM_ROUTE_DIRECT, dw, sizeof w, (const float*)dx, (const uint32_t*)dids, (float*)dy,
                       NULL, 0, NULL, &taken) != EIDM_OK || taken != EIDM_ROUTE_DIRECT) {
        printf("direct failed: %s\n", eidm_last_error());
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(yd, dy, sizeof yd, hipMemcpyDeviceToHost));
    CHECK_HIP(hipMemset(dy, 0xff, sizeof yd));
    if (eidm_matmul_id(&sh, EIDM_ROUTE_GROUPED, dw, sizeof w, (const float*)dx, (const uint32_t*)dids, (float*)dy,
                       dscr, rq.scratch_bytes, NULL, &taken) != EIDM_OK || taken != EIDM_ROUTE_GROUPED) {
        printf("grouped failed: %s\n", eidm_last_error());
        return 1;
    }
    CHECK_HIP(hipDeviceSynchronize());
    CHECK_HIP(hipMemcpy(yg, dy, sizeof yg, hipMemcpyDeviceToHost));
    if (memcmp(yd, yg, sizeof yd) != 0) {
        printf("direct and grouped differ\n");
        return 1;
    }
    double worst = 0.0;
    for (int r = 0; r < M * TOPK; ++r)
        for (int j = 0; j < N; ++j) {
            const uint16_t* wr = w + (size_t)ids[r] * N * K + (size_t)j * K;
            const float* xr = x + (size_t)(r / TOPK) * K;
            double ref = 0.0;
            for (int c = 0; c < K; ++c) ref += (double)bf16_to_f32(wr[c]) * (double)xr[c];
            const double err = fabs((double)yd[r * N + j] - ref) / fmax(1.0, fabs(ref));
            if (err > worst) worst = err;
        }
    printf("worst %.3e\n", worst);
    hipFree(dw);
    hipFree(dx);
    hipFree(dids);
    hipFree(dy);
    hipFree(dscr);
    return worst <= 2e-5 ? 0 : 1;
}
