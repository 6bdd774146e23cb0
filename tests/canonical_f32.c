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
#include <stdint.h>
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

int canonical_matmul_id(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                        uint32_t n_experts, uint64_t stride, int layout, const uint8_t* w,
                        const float* x, const uint32_t* ids, float* y) {
    int size = dtype == 0 ? 4 : 2;
    uint64_t rows = (uint64_t)m * top_k;
    uint32_t granules = ((k + 127) / 128) * 16;
    for (uint64_t r = 0; r < rows; ++r) {
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
    return 0;
}
