// moe_direct.hip -- the whole routed path for small batches in one kernel:
// route -> Direct expert-ID matmul -> gate-weighted combine.
//
// A block is one token t and one group of 4*C output columns, with one
// wavefront per slot s < top_k:
//   * the block scores token t once (each expert's sigmoid by one thread,
//     into LDS); every wavefront then runs the router's selection
//     (route_wave.hpp, the router kernel's own code) up to pick s, its
//     expert; the last wavefront runs all top_k picks and forms the gates,
//     so picks and gates are bit for bit the router kernel's (with split
//     roles the first slot takes the best of the scoring wavefronts' best
//     entries, which is the selection's first pick);
//   * the wavefronts start their weight streams one pick (about 0.2 us)
//     apart, which measured faster than starting them together;
//   * it computes its routed row t*top_k+s over the block's columns exactly
//     as the Direct kernel does (direct_columns), and stores y;
//   * the top_k rows of the block's columns meet in LDS and one wavefront
//     adds them with the combine kernel's arithmetic (f32 fma from +0, slot
//     order), so out is bit for bit what the three-kernel path gives.
// This removes two launches and the y round trip from a decode step, whose
// time is otherwise a few microseconds of routing and combining on top of
// the weight stream.
//
// cortiq-engine 0.7.7, src/mimo_moe.rs, Dynamic::run: routing, one expert
// product per pick, and the weighted sum of the picks, per token.
#include <type_traits>

#include "direct_wave.hpp"
#include "route_wave.hpp"

#ifndef EIDM_MOE_C
#define EIDM_MOE_C 2
#endif
#ifndef EIDM_MOE_DEPTH
#define EIDM_MOE_DEPTH 8
#endif

namespace eidm {
namespace {

template <int DT, int C, int D, int NV, int MAXW, bool XS, bool WHOLE, bool SPLIT>
__global__ __launch_bounds__(64 * MAXW) void moe_direct_kernel(MatmulArgs a, const float* __restrict__ logits,
                                                                const float* __restrict__ bias, int renormalize,
                                                                uint32_t* __restrict__ ids,
                                                                float* __restrict__ gates,
                                                                float* __restrict__ out, int cols_per_block) {
    constexpr bool split_roles = SPLIT;
    __shared__ float ys[MAXW][4 * C];
    __shared__ float gate_s[MAXW];
    __shared__ float rs_s[64 * NV];        // the token's router entries
    __shared__ uint32_t rs_code[64 * NV];
    __shared__ uint32_t first_code[NV], first_idx[NV];  // each scoring wavefront's best entry
    extern __shared__ __align__(16) float xs[];  // token t's activation row (XS)
    const int lane = threadIdx.x & 63;
    const int slot = threadIdx.x >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int n = (int)a.n;
    const uint32_t top_k = a.top_k;
    const uint32_t col_blocks = (a.n + cols_per_block - 1) / cols_per_block;
    const uint32_t t = blockIdx.x / col_blocks;
    const int col0 = (int)(blockIdx.x % col_blocks) * cols_per_block;
    const int col_end = min(col0 + cols_per_block, n);

    // The router entries (computed once per block) and the activation row
    // land in LDS under one barrier.  A thread's loads complete in order, so
    // the sigmoids must not queue behind the activation copy:
    //   * split_roles (the block has at least twice as many threads as
    //     router entries): the first 64*NV threads score one expert each and
    //     the others copy the activation row, so each waits for its own
    //     loads only;
    //   * otherwise every thread requests its router inputs first and its
    //     share of the copy after them, and the row arrives while the
    //     sigmoids are computed.
    const float* lrow = logits + (size_t)t * a.n_experts;
    XStage xst;
    if constexpr (SPLIT) {
        constexpr int NE = 64 * NV;
        const int tid = (int)threadIdx.x;
        if (tid < NE) {  // whole wavefronts
            const uint32_t ee = min((uint32_t)tid, a.n_experts - 1);
            const float lg = lrow[ee];
            const float bs = bias ? bias[ee] : 0.0f;
            float sv = 0.0f;
            uint32_t code = 0;
            if ((uint32_t)tid < a.n_experts) route_entry(lg, bs, sv, code);
            rs_s[tid] = sv;
            rs_code[tid] = code;
            // this wavefront's best entry (the highest code, the lowest
            // expert index among equals), for the first pick
            const uint32_t best = wave_max_u32(code);
            const uint64_t hit = __ballot(code == best);
            if ((tid & 63) == 0) {
                first_code[tid >> 6] = best;
                first_idx[tid >> 6] = (uint32_t)(tid & ~63) + (uint32_t)__builtin_ctzll(hit);
            }
        } else if constexpr (XS) {
            const int count = (int)blockDim.x - NE;
            xstage_issue_by(a.input + (size_t)t * a.k, (int)a.k, tid - NE, count, xst);
            xstage_store_by(xs, (int)a.k, tid - NE, count, xst);
        }
    } else {
        RouteInputs<NV> rin;
        route_inputs_issue<NV>(lrow, bias, a.n_experts, rin);
        if constexpr (XS) {
            __builtin_amdgcn_sched_barrier(0);
            xstage_issue(a.input + (size_t)t * a.k, (int)a.k, xst);
            __builtin_amdgcn_sched_barrier(0);
        }
        route_inputs_score<NV>(rin, a.n_experts, rs_s, rs_code);
        if constexpr (XS) xstage_store(xs, (int)a.k, xst);
    }
    __syncthreads();

    // every wavefront runs the selection up to its own pick; the last one
    // runs all top_k picks and forms the gates.  With split roles the first
    // pick is the best of the scoring wavefronts' best entries (the first
    // wavefront, lowest expert indices, wins among equal codes), so the
    // first slot's wavefront starts streaming without scanning the entries.
    uint32_t e;
    if (split_roles && slot == 0 && top_k > 1) {
        uint32_t bc = first_code[0], bi = first_idx[0];
#pragma unroll
        for (int w = 1; w < NV; ++w) {
            const uint32_t c = first_code[w];
            if (c > bc) {
                bc = c;
                bi = first_idx[w];
            }
        }
        e = bi;
    } else {
        RouteScores<NV> sc;
        route_scores_lds<NV>(rs_s, rs_code, sc);
        uint32_t pick;
        float score;
        const float sum = route_select<NV>(sc, (uint32_t)slot + 1, pick, score);
        if (slot == (int)top_k - 1) {
            const float gate = renormalize ? __fdiv_rn(score, sum) : score;
            if (lane < (int)top_k) {
                gate_s[lane] = gate;
                if (col0 == 0) {
                    ids[(size_t)t * top_k + lane] = pick;
                    gates[(size_t)t * top_k + lane] = gate;
                }
            }
        }
        e = (uint32_t)__builtin_amdgcn_readlane((int)pick, slot);
    }
    const uint32_t r = t * top_k + (uint32_t)slot;

    float v[C];
    bool cvalid[C];
    direct_columns<DT, C, D, true, XS ? kXInLds : kXFromMemory, WHOLE>(a, r, e, col0, col_end, v, cvalid, xs,
                                                                         nullptr);
    if (b == 0) {
        float* yrow = a.output + (size_t)r * a.n;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            if (cvalid[c]) yrow[col0 + 4 * c + q] = v[c];
            ys[slot][4 * c + q] = v[c];
        }
    }
    __syncthreads();
    if (slot == 0 && col0 + lane < col_end) {
        float acc = 0.0f;
        for (uint32_t s = 0; s < top_k; ++s) acc = __builtin_fmaf(gate_s[s], ys[s][lane], acc);
        out[(size_t)t * a.n + col0 + lane] = acc;
    }
}

// Ring depth: 16 wavefronts per block leave 128 VGPRs per lane, so the
// 16-slot blocks keep fewer weight rounds in flight.
template <int DT, int MAXW>
constexpr int moe_depth() {
    return MAXW <= 8 ? EIDM_MOE_DEPTH : (DT == kDtypeF32 ? 3 : 5);
}

// Columns per block.  The weight stream runs at a per-CU rate, so the
// blocks (one per CU at a time) should cover the CUs evenly: take the width
// in [max_cols/2, max_cols] whose block count wastes the least of the last
// wave of blocks (time ~ ceil(blocks / CUs) x width), the widest on ties.
// Decode (n = 1536, m = 1) on 256 CUs: 6 columns, 256 blocks.
int moe_cols_per_block(uint32_t n, uint32_t m, int max_cols, int device_cus) {
    const uint64_t cus = device_cus > 0 ? (uint64_t)device_cus : 256;
    int best = max_cols;
    uint64_t best_cost = ~0ull;
    for (int cb = max_cols; cb >= (max_cols + 1) / 2; --cb) {
        const uint64_t blocks = (uint64_t)((n + cb - 1) / cb) * m;
        const uint64_t cost = (blocks + cus - 1) / cus * (uint64_t)cb;
        if (cost < best_cost) {
            best_cost = cost;
            best = cb;
        }
    }
    return best;
}

template <int DT, int NV, int MAXW>
hipError_t launch_cfg(const MatmulArgs& a, const float* logits, const float* bias, int renormalize,
                      uint32_t* ids, float* gates, float* out, int device_cus, hipStream_t stream) {
    constexpr int C = EIDM_MOE_C;
    const int cb = moe_cols_per_block(a.n, a.m, 4 * C, device_cus);
    const uint32_t col_blocks = (a.n + cb - 1) / cb;
    const dim3 grid(col_blocks * a.m);
    constexpr int D = moe_depth<DT, MAXW>();
    // with one activation row per token, the block's wavefronts share it
    // through LDS when they can stage it in one pass (by the threads that
    // score no expert, when there are at least as many of those)
    const uint32_t threads = 64 * a.top_k;
    const int split = threads >= 2u * 64 * NV ? 1 : 0;
    const bool xs = a.layout == 0 && a.vec && direct_xstage_fits(a.k, split ? threads - 64 * NV : threads);
    // whole 128-element rounds (decode's k = 4096): a build without the
    // masked tail rounds
    const bool whole = xs && a.k % kRoundK == 0;
    auto go = [&](auto xsc, auto wholec, auto splitc) {
        constexpr bool X = decltype(xsc)::value, WH = decltype(wholec)::value, SP = decltype(splitc)::value;
        hipLaunchKernelGGL((moe_direct_kernel<DT, C, D, NV, MAXW, X, WH, SP>), grid, dim3(threads),
                           X ? (size_t)a.k * 4 : 0, stream, a, logits, bias, renormalize, ids, gates, out, cb);
    };
    using T = std::true_type;
    using F = std::false_type;
    if (split) {
        if (whole) go(T{}, T{}, T{});
        else if (xs) go(T{}, F{}, T{});
        else go(F{}, F{}, T{});
    } else {
        if (whole) go(T{}, T{}, F{});
        else if (xs) go(T{}, F{}, F{});
        else go(F{}, F{}, F{});
    }
    return launched(EIDM_KERNEL_FUSED_DECODE, grid.x, threads, xs ? a.k * 4 : 0);
}

template <int DT>
hipError_t launch_dt(const MatmulArgs& a, const float* logits, const float* bias, int renormalize,
                     uint32_t* ids, float* gates, float* out, int device_cus, hipStream_t stream) {
    if (a.n_experts <= 256) {
        if (a.top_k <= 8) return launch_cfg<DT, 4, 8>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
        return launch_cfg<DT, 4, 16>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
    }
    if (a.top_k <= 8) return launch_cfg<DT, 32, 8>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
    return launch_cfg<DT, 32, 16>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
}

}  // namespace

bool moe_direct_supported(uint32_t top_k, uint32_t n_experts) {
    return top_k >= 1 && top_k <= kMaxMoeDirectTopK && n_experts <= kMaxExperts;
}

hipError_t launch_moe_direct(const MatmulArgs& a, const float* logits, const float* bias, int renormalize,
                             uint32_t* ids, float* gates, float* out, int device_cus, hipStream_t stream) {
    switch (a.dtype) {
    case kDtypeF32: return launch_dt<kDtypeF32>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
    case kDtypeF16: return launch_dt<kDtypeF16>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
    case kDtypeBF16: return launch_dt<kDtypeBF16>(a, logits, bias, renormalize, ids, gates, out, device_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace eidm
