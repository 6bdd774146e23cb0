// combine.hip -- gate-weighted sum over the top_k slots of each token.
//
// cortiq-engine 0.7.7, src/mimo_moe.rs, Dynamic::run and run_rows: every
// pick's expert output is scaled by its final weight and the picks are
// summed; hf2q dense_ffn_arena.rs, MoeFfnArena: ids/weights are
// [seq*topk] and the expert outputs [seq*topk, h] feed a weighted reduce to
// [seq, h].
//
//   out[t, j] = sum_s gates[t, s] * y[t*top_k + s, j]   (f32 fma from +0, s ascending)
//
// Memory bound: each thread owns 4 consecutive columns of one token and
// streams the token's top_k y rows with 16-byte loads.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

__global__ __launch_bounds__(256) void combine_kernel(uint32_t m, uint32_t top_k, uint32_t n,
                                                      const float* __restrict__ y,
                                                      const float* __restrict__ gates,
                                                      float* __restrict__ out, int vec) {
    const uint32_t quads = (n + 3) / 4;
    const uint64_t total = (uint64_t)m * quads;
    for (uint64_t idx = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; idx < total;
         idx += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t t = (uint32_t)(idx / quads);
        const uint32_t j = (uint32_t)(idx % quads) * 4;
        const float* g = gates + (size_t)t * top_k;
        const float* yt = y + (size_t)t * top_k * n;
        if (vec) {
            float4 acc = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            for (uint32_t s = 0; s < top_k; ++s) {
                const float gs = g[s];
                // y is read once: non-temporal loads (3% faster than cached ones)
                const f32x4 v4 = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(yt + (size_t)s * n + j));
                const float4 v = make_float4(v4[0], v4[1], v4[2], v4[3]);
                acc.x = __builtin_fmaf(gs, v.x, acc.x);
                acc.y = __builtin_fmaf(gs, v.y, acc.y);
                acc.z = __builtin_fmaf(gs, v.z, acc.z);
                acc.w = __builtin_fmaf(gs, v.w, acc.w);
            }
            *reinterpret_cast<float4*>(out + (size_t)t * n + j) = acc;
        } else {
            for (uint32_t jj = j; jj < j + 4 && jj < n; ++jj) {
                float acc = 0.0f;
                for (uint32_t s = 0; s < top_k; ++s)
                    acc = __builtin_fmaf(g[s], yt[(size_t)s * n + jj], acc);
                out[(size_t)t * n + jj] = acc;
            }
        }
    }
}

}  // namespace

hipError_t launch_combine(uint32_t m, uint32_t top_k, uint32_t n, const float* y,
                          const float* gates, float* out, hipStream_t stream) {
    const int vec = (n % 4 == 0) && (reinterpret_cast<uintptr_t>(y) % 16 == 0) &&
                    (reinterpret_cast<uintptr_t>(out) % 16 == 0);
    const uint64_t work = (uint64_t)m * ((n + 3) / 4);
    uint64_t blocks = (work + 255) / 256;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(combine_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, m, top_k, n,
                       y, gates, out, vec);
    return launched(EIDM_KERNEL_COMBINE, (uint32_t)blocks, 256, 0);
}

}  // namespace eidm
