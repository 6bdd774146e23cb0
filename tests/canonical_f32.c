/*
 * canonical_f32.c -- test helper: the expert-ID matmul evaluated on the CPU
 * in f32 in exactly the fixed reduction order that include/eidm.h documents
 * for both GPU routes (granules of 8 along k, granule g in slice g mod 16,
 * each slice an ascending chain of f32 fma from +0, slice sums paired
 * (s, s+8), (s, s+4), (s, s+2), (s, s+1)).  The GPU output must equal it bit
 * for bit.  It is not the oracle (which sums exactly, in double) and shares
 * nothing with the HIP sources.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

static float widen(int dtype, const uint8_t* p) {
    if (dtype == 0) {
        float f;
        memcpy(&f, p, 4);
        return f;
    }
    uint16_t h;
    memcpy(&h, p, 2);
    if (dtype == 2) {
        uint32_t u = (uint32_t)h << 16;
        float f;
        memcpy(&f, &u, 4);
        return f;
    }
    int s = h >> 15, e = (h >> 10) & 31, fr = h & 1023;
    float v = e == 0 ? ldexpf((float)fr, -24) : e == 31 ? (fr ? NAN : INFINITY) : ldexpf(1.0f + fr / 1024.0f, e - 15);
    return s ? -v : v;
}

/* routed rows [r0, r1) */
static void canonical_rows(int dtype, uint32_t n, uint32_t k, uint32_t top_k, uint32_t n_experts, uint64_t stride,
                           int layout, const uint8_t* w, const float* x, const uint32_t* ids, float* y, uint64_t r0,
                           uint64_t r1) {
    int size = dtype == 0 ? 4 : 2;
    uint32_t granules = ((k + 127) / 128) * 16;
    for (uint64_t r = r0; r < r1; ++r) {
        uint32_t e = ids[r];
        for (uint32_t j = 0; j < n; ++j) {
            if (e >= n_experts) {
                y[r * n + j] = NAN;
                continue;
            }
            const float* xr = layout == 1 ? x + r * k : x + (r / top_k) * k;
            const uint8_t* wr = w + (uint64_t)e * stride + (uint64_t)j * k * size;
            float s[16];
            for (int b = 0; b < 16; ++b) {
                float acc = 0.0f;
                for (uint32_t g = b; g < granules; g += 16)
                    for (int i = 0; i < 8; ++i) {
                        uint32_t c = g * 8 + i;
                        float wv = c < k ? widen(dtype, wr + (uint64_t)c * size) : 0.0f;
                        float xv = c < k ? xr[c] : 0.0f;
                        acc = fmaf(wv, xv, acc);
                    }
                s[b] = acc;
            }
            for (int b = 0; b < 8; ++b) s[b] = s[b] + s[b + 8];
            for (int b = 0; b < 4; ++b) s[b] = s[b] + s[b + 4];
            for (int b = 0; b < 2; ++b) s[b] = s[b] + s[b + 2];
            y[r * n + j] = s[0] + s[1];
        }
    }
}

int canonical_matmul_id(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                        uint32_t n_experts, uint64_t stride, int layout, const uint8_t* w,
                        const float* x, const uint32_t* ids, float* y) {
    canonical_rows(dtype, n, k, top_k, n_experts, stride, layout, w, x, ids, y, 0, (uint64_t)m * top_k);
    return 0;
}

/* The same values with the loops reordered for speed at full sizes: the
 * routed rows grouped by expert, experts handed out one at a time to `threads`
 * threads (the caller's among them), and each weight row widened once per expert.  Every output is
 * still the one chain-and-tree evaluation above, so the bits are unchanged. */
struct Shared {
    int dtype, layout;
    uint32_t n, k, top_k, n_experts;
    uint64_t stride;
    const uint8_t* w;
    const float* x;
    const uint64_t* start;  /* rows of expert e: order[start[e] .. start[e+1]) */
    const uint64_t* order;
    float* y;
    uint32_t next;          /* next expert to take */
};

static void* run_experts(void* arg) {
    struct Shared* sh = (struct Shared*)arg;
    int size = sh->dtype == 0 ? 4 : 2;
    uint32_t k = sh->k, n = sh->n;
    uint32_t granules = ((k + 127) / 128) * 16;
    float* wv = (float*)calloc((size_t)granules * 8, sizeof(float));
    float* xv = (float*)calloc((size_t)granules * 8, sizeof(float));
    if (!wv || !xv) {
        free(wv);
        free(xv);
        return (void*)1;
    }
    for (;;) {
        uint32_t e = __atomic_fetch_add(&sh->next, 1, __ATOMIC_RELAXED);
        if (e >= sh->n_experts) break;
        uint64_t a = sh->start[e], b = sh->start[e + 1];
        if (a == b) continue;
        for (uint32_t j = 0; j < n; ++j) {
            const uint8_t* wr = sh->w + (uint64_t)e * sh->stride + (uint64_t)j * k * size;
            for (uint32_t c = 0; c < k; ++c) wv[c] = widen(sh->dtype, wr + (uint64_t)c * size);
            for (uint64_t q = a; q < b; ++q) {
                uint64_t r = sh->order[q];
                const float* xr = sh->layout == 1 ? sh->x + r * k : sh->x + (r / sh->top_k) * k;
                memcpy(xv, xr, (size_t)k * sizeof(float));
                float s[16];
                for (int t = 0; t < 16; ++t) {
                    float acc = 0.0f;
                    for (uint32_t g = t; g < granules; g += 16)
                        for (int i = 0; i < 8; ++i) acc = fmaf(wv[g * 8 + i], xv[g * 8 + i], acc);
                    s[t] = acc;
                }
                for (int t = 0; t < 8; ++t) s[t] = s[t] + s[t + 8];
                for (int t = 0; t < 4; ++t) s[t] = s[t] + s[t + 4];
                for (int t = 0; t < 2; ++t) s[t] = s[t] + s[t + 2];
                sh->y[r * n + j] = s[0] + s[1];
            }
        }
    }
    free(wv);
    free(xv);
    return 0;
}

int canonical_matmul_id_threads(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k, uint32_t n_experts,
                                uint64_t stride, int layout, const uint8_t* w, const float* x, const uint32_t* ids,
                                float* y, int threads) {
    if (threads < 1) threads = 1;
    if (threads > 256) threads = 256;
    uint64_t rows = (uint64_t)m * top_k;
    uint64_t* start = (uint64_t*)calloc((size_t)n_experts + 2, sizeof(uint64_t));
    uint64_t* order = (uint64_t*)malloc((size_t)(rows ? rows : 1) * sizeof(uint64_t));
    if (!start || !order) {
        free(start);
        free(order);
        return -1;
    }
    /* counting sort of the routed rows by expert; rows naming no expert are NaN */
    for (uint64_t r = 0; r < rows; ++r)
        if (ids[r] < n_experts) start[ids[r] + 1]++;
    for (uint32_t e = 0; e < n_experts; ++e) start[e + 1] += start[e];
    uint64_t* fill = (uint64_t*)malloc(((size_t)n_experts + 1) * sizeof(uint64_t));
    if (!fill) {
        free(start);
        free(order);
        return -1;
    }
    memcpy(fill, start, ((size_t)n_experts + 1) * sizeof(uint64_t));
    for (uint64_t r = 0; r < rows; ++r) {
        if (ids[r] < n_experts) {
            order[fill[ids[r]]++] = r;
        } else {
            for (uint32_t j = 0; j < n; ++j) y[r * n + j] = NAN;
        }
    }
    free(fill);
    struct Shared sh = {dtype, layout, n, k, top_k, n_experts, stride, w, x, start, order, y, 0};
    pthread_t tid[256];
    int created[256];
    int rc = 0;
    for (int t = 0; t + 1 < threads; ++t) created[t] = pthread_create(&tid[t], 0, run_experts, &sh) == 0;
    if (run_experts(&sh)) rc = -1;  /* the caller's thread takes experts too */
    for (int t = 0; t + 1 < threads; ++t) {
        void* out = 0;
        if (created[t]) pthread_join(tid[t], &out);
        if (out) rc = -1;
    }
    free(start);
    free(order);
    return rc;
}
