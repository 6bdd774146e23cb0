// direct_wave.hpp -- one wavefront of the Direct form: 4*C output columns of
// one routed row, streaming that expert's weight rows from HBM once.  Used by
// the Direct kernel and by the fused decode kernel.
//
// The work is a weight stream (HBM-bound at small m), so it is built around
// keeping many 16-byte loads in flight and never waiting for more than the
// oldest one:
//   * the round loop is a ring of D register slots: round g is consumed while
//     rounds g+1 .. g+D-1 are in flight, and round g+D is requested as soon as
//     slot g is free;
//   * a slot holds this lane's weight granules and its slice's activation
//     granule (the four lanes of one matrix-core block read the same 32
//     bytes, which the L2 serves), so the loop has one in-order load stream
//     and no LDS, barriers or per-lane branches;
//   * columns past the computed ones re-read the first one and rows are
//     whole granules, so every vector round issues the same loads in every
//     lane.
// Per round (128 k), lane 4b+q (slice b, column q) holds one 8-element weight
// granule per column group; the lanes with q == 0 feed the activation as the
// only valid A-row of the matrix-core block.  The k tail (and rows that are
// not 16-byte aligned) take masked loads after the ring.
#pragma once

#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {

// 16-byte pieces of one weight granule: 1 for 16-bit types, 2 for f32.
template <int DT> struct DirectPieces { static constexpr int value = DtypeSize<DT>::value / 2; };

typedef unsigned int u32x4_t __attribute__((ext_vector_type(4)));

template <int DT>
__device__ __forceinline__ void direct_widen(const u32x4_t (&p)[DirectPieces<DT>::value], float (&w)[kGranule]) {
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
struct DirectSlot {
    u32x4_t w[C][DirectPieces<DT>::value];
    f32x4 x[2];
};

// Columns col0 .. col0+4C-1 of routed row r, whose expert is e (< n_experts);
// the columns from col_end on (col0 < col_end <= n) are not computed: their
// lanes re-read column col0, so every lane issues the same loads.
// On return lane q of slice 0 (lanes 0..3) holds in v[c] the output of
// column col0 + 4c + q (every other lane holds the same totals of its own
// slice group); cvalid[c] says whether that column is one of the computed.
template <int DT, int C, int D, bool NT>
__device__ __forceinline__ void direct_columns(const MatmulArgs& a, uint32_t r, uint32_t e, int col0,
                                               int col_end, float (&v)[C], bool (&cvalid)[C]) {
    constexpr int S = DtypeSize<DT>::value;
    constexpr int NP = DirectPieces<DT>::value;
    const int lane = threadIdx.x & 63;
    const int b = lane >> 2, q = lane & 3;
    const int k = (int)a.k;

    const uint32_t xr = a.layout == 1 ? r : r / a.top_k;
    const float* xrow = a.input + (size_t)xr * a.k;
    const float* xlane = xrow + b * kGranule;
    const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;

    const uint8_t* wrow[C];  // this lane's granule of round 0, per column group
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int col = col0 + 4 * c + q;
        cvalid[c] = col < col_end;
        wrow[c] = wexp + (size_t)(cvalid[c] ? col : col0) * a.k * S + (size_t)b * kGranule * S;
    }

    const int rounds = (k + kRoundK - 1) / kRoundK;
    // rounds whose granules are whole and 16-byte aligned: the pipelined path
    const int full = a.vec ? k / kRoundK : 0;

    auto fetch = [&](int g, DirectSlot<DT, C>& s) {
#pragma unroll
        for (int c = 0; c < C; ++c)
#pragma unroll
            for (int i = 0; i < NP; ++i) {
                const u32x4_t* p = reinterpret_cast<const u32x4_t*>(wrow[c] + (size_t)g * kRoundK * S) + i;
                if constexpr (NT)
                    s.w[c][i] = __builtin_nontemporal_load(p);  // weights are read once per call
                else
                    s.w[c][i] = *p;
            }
        s.x[0] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK);
        s.x[1] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK + 4);
    };

    f32x4 acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    auto consume = [&](const DirectSlot<DT, C>& s) {
        float x[kGranule];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = q == 0 ? s.x[0][i] : 0.0f;
            x[4 + i] = q == 0 ? s.x[1][i] : 0.0f;
        }
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c) direct_widen<DT>(s.w[c], w[c]);
#pragma unroll
        for (int i = 0; i < kGranule; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = mfma_step(x[i], w[c][i], acc[c]);
    };

    if (full > 0) {
        // request the first D rounds (past the last vector round the last one
        // is requested again: only when k < D*128)
        DirectSlot<DT, C> ring[D];
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
    for (int c = 0; c < C; ++c) v[c] = slice_tree(acc[c][0]);
}

}  // namespace eidm
