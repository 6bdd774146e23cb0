// route_wave.hpp -- one token's sigmoid + selection-bias top-k on one
// wavefront; used by the router kernel and by the fused decode kernel, so
// both pick the same experts with the same gates bit for bit.
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
#pragma once

#include "eidm_device.hpp"

namespace eidm {

// Rank code of a selection score: larger score -> larger code; -0 as +0; a
// NaN ranks below every number (code 1); 0 is left for "taken / no such
// expert".  Equal codes are equal scores, which go to the lower expert index.
__device__ __forceinline__ uint32_t rank_code(float f) {
    if (f != f) return 1u;
    if (f == 0.0f) f = 0.0f;
    const uint32_t u = __float_as_uint(f);
    return ((u & 0x80000000u) ? ~u : (u | 0x80000000u)) + 1u;  // numbers: 0x00800000 .. 0xff800001
}

template <int CTRL>
__device__ __forceinline__ uint32_t dpp32(uint32_t v) {
    return (uint32_t)__builtin_amdgcn_mov_dpp((int)v, CTRL, 0xf, 0xf, false);
}

// Maximum over the wavefront: quad swaps, half-row and row mirrors (DPP), then
// the four row maxima through scalar registers.
__device__ __forceinline__ uint32_t wave_max_u32(uint32_t v) {
    v = max(v, dpp32<0xb1>(v));   // quad_perm [1,0,3,2]
    v = max(v, dpp32<0x4e>(v));   // quad_perm [2,3,0,1]
    v = max(v, dpp32<0x141>(v));  // row_half_mirror
    v = max(v, dpp32<0x140>(v));  // row_mirror
    const uint32_t r0 = (uint32_t)__builtin_amdgcn_readlane((int)v, 0);
    const uint32_t r1 = (uint32_t)__builtin_amdgcn_readlane((int)v, 16);
    const uint32_t r2 = (uint32_t)__builtin_amdgcn_readlane((int)v, 32);
    const uint32_t r3 = (uint32_t)__builtin_amdgcn_readlane((int)v, 48);
    return max(max(r0, r1), max(r2, r3));
}

// One token's scores on the calling wavefront: expert v*64 + lane in slot v.
template <int NV>
struct RouteScores {
    float s[NV];         // sigmoid(logit), rounded to f32
    uint32_t code[NV];   // rank code of s + bias (0 once picked, or past n_experts)
};

// One expert's entry: s = sigmoid(logit) in double rounded once to f32, and
// the rank code of s + bias.
__device__ __forceinline__ void route_entry(float logit, float b, float& s, uint32_t& code) {
    s = (float)(1.0 / (1.0 + exp(-(double)logit)));
    code = rank_code(s + b);
}

// The token's entries computed by the calling wavefront alone.
template <int NV>
__device__ __forceinline__ void route_scores(const float* __restrict__ lrow, const float* __restrict__ bias,
                                             uint32_t n_experts, RouteScores<NV>& sc) {
    const int lane = threadIdx.x & 63;
    // all loads first (lanes past n_experts >= 1 re-read the last expert), so
    // the wavefront waits for memory once
    float lg[NV], bs[NV];
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint32_t e = min((uint32_t)v * 64 + lane, n_experts - 1);
        lg[v] = lrow[e];
        bs[v] = bias ? bias[e] : 0.0f;
    }
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        const uint32_t e = (uint32_t)v * 64 + lane;
        sc.s[v] = 0.0f;
        sc.code[v] = 0;
        if (e < n_experts) route_entry(lg[v], bs[v], sc.s[v], sc.code[v]);
    }
}

// The token's entries computed once per block: thread i takes experts
// i, i + blockDim.x, ... and writes them to LDS (s_lds, code_lds: 64*NV
// entries, those past n_experts as 0).  After a barrier each wavefront reads
// its copy with route_scores_lds.  The double-precision sigmoid is the
// router's costliest step, so a block of W wavefronts spreads it W ways
// instead of repeating it in every wavefront.
// The block's share of one token's router inputs, requested but not yet
// waited for: thread i holds experts i, i + blockDim.x, ... (64*NV slots).
template <int NV>
struct RouteInputs {
    float lg[NV], bs[NV];
};

template <int NV>
__device__ __forceinline__ void route_inputs_issue(const float* __restrict__ lrow, const float* __restrict__ bias,
                                                   uint32_t n_experts, RouteInputs<NV>& in) {
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        if (i * nt < 64 * NV) {  // block-uniform
            const uint32_t e = min((uint32_t)(i * nt + tid), n_experts - 1);
            in.lg[i] = lrow[e];
            in.bs[i] = bias ? bias[e] : 0.0f;
        }
    }
}

// The sigmoids and rank codes of the inputs into LDS (s_lds, code_lds: 64*NV
// entries, those past n_experts as 0).
template <int NV>
__device__ __forceinline__ void route_inputs_score(const RouteInputs<NV>& in, uint32_t n_experts, float* s_lds,
                                                   uint32_t* code_lds) {
    const int tid = (int)threadIdx.x, nt = (int)blockDim.x;
#pragma unroll
    for (int i = 0; i < NV; ++i) {
        const int e = i * nt + tid;
        if (i * nt < 64 * NV && e < 64 * NV) {
            float s = 0.0f;
            uint32_t code = 0;
            if ((uint32_t)e < n_experts) route_entry(in.lg[i], in.bs[i], s, code);
            s_lds[e] = s;
            code_lds[e] = code;
        }
    }
}

template <int NV>
__device__ __forceinline__ void route_scores_shared(const float* __restrict__ lrow, const float* __restrict__ bias,
                                                    uint32_t n_experts, float* s_lds, uint32_t* code_lds) {
    RouteInputs<NV> in;
    route_inputs_issue<NV>(lrow, bias, n_experts, in);
    route_inputs_score<NV>(in, n_experts, s_lds, code_lds);
}

template <int NV>
__device__ __forceinline__ void route_scores_lds(const float* s_lds, const uint32_t* code_lds, RouteScores<NV>& sc) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int v = 0; v < NV; ++v) {
        sc.s[v] = s_lds[v * 64 + lane];
        sc.code[v] = code_lds[v * 64 + lane];
    }
}

// Picks 0 .. rounds-1 (largest score first, ties to the lower index): lane
// j < rounds receives pick j's expert and score.  Returns the sum of the
// picks' scores added in pick order (the same value in every lane).
template <int NV>
__device__ __forceinline__ float route_select(RouteScores<NV>& sc, uint32_t rounds, uint32_t& id, float& score) {
    const int lane = threadIdx.x & 63;
    uint32_t my_id = 0;
    float my_s = 0.0f, sum = 0.0f;
    for (uint32_t j = 0; j < rounds; ++j) {
        uint32_t best = 0;
#pragma unroll
        for (int v = 0; v < NV; ++v) best = max(best, sc.code[v]);
        best = wave_max_u32(best);  // wave-uniform
        // the lowest expert index holding the best code
        uint32_t e = 0xffffffffu;
#pragma unroll
        for (int v = NV - 1; v >= 0; --v) {
            const uint64_t hit = __ballot(sc.code[v] == best);
            if (hit) e = (uint32_t)v * 64 + (uint32_t)__builtin_ctzll(hit);
        }
        const int owner = (int)(e & 63u), slot = (int)(e >> 6);
        float mine = 0.0f;
#pragma unroll
        for (int v = 0; v < NV; ++v) {
            if (v == slot) {
                mine = sc.s[v];
                if (lane == owner) sc.code[v] = 0;
            }
        }
        const float sw = __builtin_bit_cast(float, __builtin_amdgcn_readlane(__builtin_bit_cast(int, mine), owner));
        sum += sw;  // pick order, identical in every lane
        if (lane == (int)j) {
            my_id = e;
            my_s = sw;
        }
    }
    id = my_id;
    score = my_s;
    return sum;
}

// Route one token (logits row `lrow`, n_experts <= 64*NV) on the calling
// wavefront.  Afterwards lane j < top_k holds pick j: its expert in `id` and
// its gate in `gate` (s / sum of the picks' s when renormalising, else s).
template <int NV>
__device__ __forceinline__ void route_token(const float* __restrict__ lrow, const float* __restrict__ bias,
                                            uint32_t n_experts, uint32_t top_k, int renormalize,
                                            uint32_t& id, float& gate) {
    RouteScores<NV> sc;
    route_scores<NV>(lrow, bias, n_experts, sc);
    float s;
    const float sum = route_select<NV>(sc, top_k, id, s);
    gate = renormalize ? __fdiv_rn(s, sum) : s;
}

}  // namespace eidm
