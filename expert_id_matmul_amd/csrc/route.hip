// route.hip -- sigmoid + selection-bias top-k router, one wavefront per token.
//
// cortiq-engine 0.7.7, src/mimo_moe.rs: the module doc describes top-8 of
// 256 experts chosen by sigmoid scores with a per-expert selection bias; the
// bank_tests model arch sets router_sigmoid and norm_topk_prob; Dynamic::run
// applies each pick's weight as p[e] / wsum with route scale 1.
//
//   s = sigmoid(logit) rounded to f32; sel = s + bias (f32 add);
//   picks = top_k largest sel, equal sel -> lower expert index first;
//   gate = s / (sum of the picks' s, added in slot order) when renormalising.
//
// The sigmoid is evaluated in double and rounded once to f32, so the value
// is the correctly rounded one up to the double evaluation's error; the
// selection therefore does not depend on a particular f32 exp.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

constexpr uint32_t kNone = 0xffffffffu;

// Strict total order on (key, index): larger key first, a NaN key after
// every number, equal keys (and NaN pairs) by lower index.  An empty slot
// (index kNone) ranks last.
__device__ __forceinline__ bool ranks_before(float a, uint32_t ai, float b, uint32_t bi) {
    if (ai == kNone) return false;
    if (bi == kNone) return true;
    const bool an = a != a, bn = b != b;
    if (an != bn) return bn;
    if (!an && a != b) return a > b;
    return ai < bi;
}

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, uint32_t m,
                                                    uint32_t n_experts, uint32_t top_k,
                                                    int renormalize, uint32_t* __restrict__ ids,
                                                    float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const uint32_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= m) return;
    const float* lrow = logits + (size_t)t * n_experts;

    float s[NV], sel[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint32_t e = (uint32_t)v * 64 + lane;
        s[v] = 0.0f;
        sel[v] = 0.0f;
        if (e < n_experts) {
            const double sd = 1.0 / (1.0 + exp(-(double)lrow[e]));
            s[v] = (float)sd;
            sel[v] = s[v] + (bias ? bias[e] : 0.0f);
        }
    }

    uint32_t taken = 0;  // bit v: value v of this lane already picked
    float gsum = 0.0f;
    for (uint32_t j = 0; j < top_k; ++j) {
        float bs = 0.0f;
        uint32_t bi = kNone;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            const uint32_t e = (uint32_t)v * 64 + lane;
            if (e < n_experts && !((taken >> v) & 1u) && ranks_before(sel[v], e, bs, bi)) {
                bs = sel[v];
                bi = e;
            }
        }
#pragma unroll
        for (int off = 32; off >= 1; off >>= 1) {
            const float os = __shfl_xor(bs, off);
            const uint32_t oi = __shfl_xor(bi, off);
            if (ranks_before(os, oi, bs, bi)) {
                bs = os;
                bi = oi;
            }
        }
        // every lane now holds the same winner
        const int owner = (int)(bi & 63u);
        const int slot = (int)(bi >> 6);
        float mine = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v)
            if (v == slot) mine = s[v];
        if (lane == owner) taken |= 1u << slot;
        const float sw = __shfl(mine, owner);
        if (lane == 0) {
            ids[(size_t)t * top_k + j] = bi;
            gsum += sw;
            if (gates) gates[(size_t)t * top_k + j] = sw;
        }
    }
    if (lane == 0 && gates && renormalize) {
        for (uint32_t j = 0; j < top_k; ++j) {
            float* g = gates + (size_t)t * top_k + j;
            *g = __fdiv_rn(*g, gsum);
        }
    }
}

template <int NV>
hipError_t launch_nv(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                     uint32_t top_k, int renormalize, uint32_t* ids, float* gates,
                     hipStream_t stream) {
    const dim3 grid((m + 3) / 4);
    hipLaunchKernelGGL(route_kernel<NV>, grid, dim3(256), 0, stream, logits, bias, m, n_experts,
                       top_k, renormalize, ids, gates);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_route(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                        uint32_t top_k, int renormalize, uint32_t* ids, float* gates,
                        hipStream_t stream) {
    const uint32_t nv = (n_experts + 63) / 64;
    if (nv <= 1) return launch_nv<1>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
    if (nv <= 2) return launch_nv<2>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
    if (nv <= 4) return launch_nv<4>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
    if (nv <= 8) return launch_nv<8>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
    if (nv <= 16) return launch_nv<16>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
    return launch_nv<32>(logits, bias, m, n_experts, top_k, renormalize, ids, gates, stream);
}

}  // namespace eidm
