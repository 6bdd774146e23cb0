// matmul_direct.hip -- Direct form of the expert-ID matmul: each wavefront
// computes 4*C output columns of one routed row, streaming that expert's
// weight rows from HBM once.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: fn expected_dispatches
// gives the Direct route one dispatch over (column groups) x (m*top_k routed
// rows); the value-independence theorem statement fixes what it shares with
// the grouped route.  Here a block is WAVES wavefronts of 4*C columns of one
// routed row.
//
// The work is a weight stream (HBM-bound at small m), so the kernel is built
// around keeping many 16-byte loads in flight and never waiting for more than
// the oldest one:
//   * the round loop is a ring of D register slots: round g is consumed while
//     rounds g+1 .. g+D-1 are in flight, and round g+D is requested as soon as
//     slot g is free;
//   * a slot holds this lane's weight granules and its slice's activation
//     granule (the four lanes of one matrix-core block read the same 32
//     bytes, which the L2 serves), so the loop has one in-order load stream
//     and no LDS, barriers or per-lane branches;
//   * columns past n read column 0 and rows are whole granules, so every
//     vector round issues the same loads in every lane.
// Per round (128 k), lane 4b+q (slice b, column q) holds one 8-element weight
// granule per column group; the lanes with q == 0 feed the activation as the
// only valid A-row of the matrix-core block.  The k tail (and rows that are
// not 16-byte aligned) take masked loads after the ring.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

#ifndef EIDM_DIRECT_C
#define EIDM_DIRECT_C 2
#endif
#ifndef EIDM_DIRECT_WAVES
#define EIDM_DIRECT_WAVES 2
#endif
#ifndef EIDM_DIRECT_DEPTH
#define EIDM_DIRECT_DEPTH 6
#endif
#ifndef EIDM_DIRECT_NT
#define EIDM_DIRECT_NT 1
#endif

namespace eidm {
namespace {

// 16-byte pieces of one weight granule: 1 for 16-bit types, 2 for f32.
template <int DT> struct Pieces { static constexpr int value = DtypeSize<DT>::value / 2; };

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ void widen_pieces(const u32x4 (&p)[Pieces<DT>::value], float (&w)[kGranule]) {
    if constexpr (DT == kDtypeF32) {
        w[0] = __uint_as_float(p[0].x); w[1] = __uint_as_float(p[0].y);
        w[2] = __uint_as_float(p[0].z); w[3] = __uint_as_float(p[0].w);
        w[4] = __uint_as_float(p[1].x); w[5] = __uint_as_float(p[1].y);
        w[6] = __uint_as_float(p[1].z); w[7] = __uint_as_float(p[1].w);
    } else {
        widen_pair<DT>(p[0].x, w[0], w[1]);
        widen_pair<DT>(p[0].y, w[2], w[3]);
        widen_pair<DT>(p[0].z, w[4], w[5]);
        widen_pair<DT>(p[0].w, w[6], w[7]);
    }
}

// One ring slot: this lane's weight granules for its C columns and the
// activation granule of its slice, for one round.
template <int DT, int C>
struct Slot {
    u32x4 w[C][Pieces<DT>::value];
    f32x4 x[2];
};

template <int DT, int C, int WAVES, int D>
__global__ __launch_bounds__(64 * WAVES) void direct_kernel(MatmulArgs a) {
    constexpr int S = DtypeSize<DT>::value;
    constexpr int NP = Pieces<DT>::value;

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int n = (int)a.n, k = (int)a.k;
    const uint32_t col_blocks = (a.n + 4 * C * WAVES - 1) / (4 * C * WAVES);
    const uint32_t r = blockIdx.x / col_blocks;
    const int col0 = ((int)(blockIdx.x % col_blocks) * WAVES + wave) * (4 * C);
    if (col0 >= n) return;  // wave-uniform; nothing below synchronises the block
    float* yrow = a.output + (size_t)r * a.n;

    const uint32_t e = a.ids[r];
    if (e >= a.n_experts) {  // no weights for this row: quiet NaN
        if (lane < 4 * C && col0 + lane < n) yrow[col0 + lane] = quiet_nan();
        return;
    }
    const uint32_t xr = a.layout == 1 ? r : r / a.top_k;
    const float* xrow = a.input + (size_t)xr * a.k;
    const float* xlane = xrow + b * kGranule;
    const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;

    const uint8_t* wrow[C];  // this lane's granule of round 0, per column group
    bool cvalid[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int col = col0 + 4 * c + q;
        cvalid[c] = col < n;
        wrow[c] = wexp + (size_t)(cvalid[c] ? col : 0) * a.k * S + (size_t)b * kGranule * S;
    }

    const int rounds = (k + kRoundK - 1) / kRoundK;
    // rounds whose granules are whole and 16-byte aligned: the pipelined path
    const int full = a.vec ? k / kRoundK : 0;

    auto fetch = [&](int g, Slot<DT, C>& s) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < NP; ++i)
            {
                const u32x4* p = reinterpret_cast<const u32x4*>(wrow[c] + (size_t)g * kRoundK * S) + i;
#if EIDM_DIRECT_NT
                s.w[c][i] = __builtin_nontemporal_load(p);  // weights are read once per call
#else
                s.w[c][i] = *p;
#endif
            }
        s.x[0] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK);
        s.x[1] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK + 4);
    };

    f32x4 acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto consume = [&](const Slot<DT, C>& s) {
        float x[kGranule];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = q == 0 ? s.x[0][i] : 0.0f;
            x[4 + i] = q == 0 ? s.x[1][i] : 0.0f;
        }
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c) widen_pieces<DT>(s.w[c], w[c]);
#pragma unroll
        for (int i = 0; i < kGranule; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = mfma_step(x[i], w[c][i], acc[c]);
    };

    if (full > 0) {
        // request the first D rounds (past the last vector round the last one
        // is requested again: only when k < D*128)
        Slot<DT, C> ring[D];
#pragma unroll
        for (int d = 0; d < D; ++d) {
            fetch(min(d, full - 1), ring[d]);
            __builtin_amdgcn_sched_barrier(0);  // issue in slot order
        }
        int g = 0;
        // steady state: every round refills its slot; the scheduling barrier
        // keeps rounds in order so each wait is only for the oldest slot
        for (; g + 2 * D <= full; g += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                consume(ring[d]);
                fetch(g + d + D, ring[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last vector rounds (slots stay in order)
#pragma unroll
        for (int j = 0; j < 2 * D; ++j) {
            const int gg = g + j;
            if (gg < full) {
                consume(ring[j % D]);
                if (gg + D < full) fetch(gg + D, ring[j % D]);
            }
        }
    }
    // rounds that need masked loads (k tail, or rows not 16-byte aligned)
    for (int g = full; g < rounds; ++g) {
        float x[kGranule];
        load_input_granule(xrow, g * kRoundK + b * kGranule, k, q == 0, false, x);
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c)
            load_weight_granule<DT>(wrow[c] - (size_t)b * kGranule * S, g * kRoundK + b * kGranule, k,
                                    cvalid[c], false, w[c]);
#pragma unroll
        for (int i = 0; i < kGranule; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = mfma_step(x[i], w[c][i], acc[c]);
    }

#pragma unroll
    for (int c = 0; c < C; ++c) {
        const float v = slice_tree(acc[c][0]);
        if (b == 0 && cvalid[c]) yrow[col0 + 4 * c + q] = v;
    }
}

template <int DT, int C, int WAVES, int D>
hipError_t launch_cfg(const MatmulArgs& a, hipStream_t stream) {
    const uint32_t cols_per_block = 4 * C * WAVES;
    const dim3 grid(((a.n + cols_per_block - 1) / cols_per_block) * (a.m * a.top_k));
    hipLaunchKernelGGL((direct_kernel<DT, C, WAVES, D>), grid, dim3(64 * WAVES), 0, stream, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const MatmulArgs& a, hipStream_t stream) {
    return launch_cfg<DT, EIDM_DIRECT_C, EIDM_DIRECT_WAVES, EIDM_DIRECT_DEPTH>(a, stream);
}

}  // namespace

hipError_t launch_direct(const MatmulArgs& a, hipStream_t stream) {
    switch (a.dtype) {
    case kDtypeF32: return launch_dt<kDtypeF32>(a, stream);
    case kDtypeF16: return launch_dt<kDtypeF16>(a, stream);
    case kDtypeBF16: return launch_dt<kDtypeBF16>(a, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace eidm
