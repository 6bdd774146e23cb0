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

// Monotone map of an f32 key to u32: larger key -> larger code, -0 as +0, a
// NaN below every number.
__device__ __forceinline__ uint32_t order_code(float f) {
    if (f != f) return 0u;
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// 64-bit rank: code in the high word, (~index) in the low word, so the
// maximum is the largest key with ties going to the lower index.  0 marks an
// expert that is taken or does not exist.
__device__ __forceinline__ uint64_t rank_of(float sel, uint32_t e) {
    return ((uint64_t)order_code(sel) << 32) | (uint64_t)(0xffffffffu - e);
}

template <int CTRL>
__device__ __forceinline__ uint64_t dpp64(uint64_t v) {
    const int lo = __builtin_amdgcn_mov_dpp((int)(uint32_t)v, CTRL, 0xf, 0xf, false);
    const int hi = __builtin_amdgcn_mov_dpp((int)(uint32_t)(v >> 32), CTRL, 0xf, 0xf, false);
    return ((uint64_t)(uint32_t)hi << 32) | (uint32_t)lo;
}

__device__ __forceinline__ uint64_t umax64(uint64_t a, uint64_t b) { return a > b ? a : b; }

__device__ __forceinline__ uint64_t readlane64(uint64_t v, int lane) {
    const uint32_t lo = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)v, lane);
    const uint32_t hi = (uint32_t)__builtin_amdgcn_readlane((int)(uint32_t)(v >> 32), lane);
    return ((uint64_t)hi << 32) | lo;
}

// Maximum over the wavefront: quad swaps, half-row and row mirrors (DPP), then
// the four row maxima through scalar registers.
__device__ __forceinline__ uint64_t wave_max(uint64_t v) {
    v = umax64(v, dpp64<0xb1>(v));   // quad_perm [1,0,3,2]
    v = umax64(v, dpp64<0x4e>(v));   // quad_perm [2,3,0,1]
    v = umax64(v, dpp64<0x141>(v));  // row_half_mirror
    v = umax64(v, dpp64<0x140>(v));  // row_mirror
    return umax64(umax64(readlane64(v, 0), readlane64(v, 16)),
                  umax64(readlane64(v, 32), readlane64(v, 48)));
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

    float s[NV];
    uint64_t key[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint32_t e = (uint32_t)v * 64 + lane;
        s[v] = 0.0f;
        key[v] = 0;
        if (e < n_experts) {
            s[v] = (float)(1.0 / (1.0 + exp(-(double)lrow[e])));
            const float sel = s[v] + (bias ? bias[e] : 0.0f);
            key[v] = rank_of(sel, e);
        }
    }

    uint32_t my_id = 0;
    float my_s = 0.0f, gsum = 0.0f;
    for (uint32_t j = 0; j < top_k; ++j) {
        uint64_t best = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) best = umax64(best, key[v]);
        best = wave_max(best);  // wave-uniform
        const uint32_t e = 0xffffffffu - (uint32_t)best;
        const int owner = (int)(e & 63u), slot = (int)(e >> 6);
        float mine = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (v == slot) {
                mine = s[v];
                if (lane == owner) key[v] = 0;
            }
        }
        const float sw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine), owner));
        gsum += sw;  // slot order, identical in every lane
        if (lane == (int)j) {
            my_id = e;
            my_s = sw;
        }
    }
    if (lane < (int)top_k) {
        ids[(size_t)t * top_k + lane] = my_id;
        if (gates) gates[(size_t)t * top_k + lane] = renormalize ? __fdiv_rn(my_s, gsum) : my_s;
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
