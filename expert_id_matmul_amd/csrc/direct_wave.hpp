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
//   * the activation row is staged once per block in LDS when the block's
//     threads can carry it in one pass (XS): its loads go out before the
//     first weight rounds and are stored after them, so the copy hides under
//     the ring's fill, and the loop's only memory requests are weights.
//     Otherwise a slot also holds its slice's activation granule (the four
//     lanes of one slice read the same 32 bytes, which the cache serves);
//     either way the loop has one in-order load stream and no per-lane
//     branches;
//   * columns past the computed ones re-read the first one and rows are
//     whole granules, so every vector round issues the same loads in every
//     lane.
// Per round (128 k), lane 4b+q (slice b, column q) holds one 8-element weight
// granule per column group and accumulates its own (slice, column) element
// with vector fmas: with a single activation row, three of the four A-rows
// of a 4x4x1 matrix-core block would be idle, and the vector step costs half
// the issue cycles of the matrix-core one for the same bits (the step is
// described with the canonical order).  The k tail (and rows that are not
// 16-byte aligned) take masked loads after the ring.
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
// activation granule of its slice, for one round (the latter unused when the
// activation row sits in LDS).
template <int DT, int C>
struct DirectSlot {
    u32x4_t w[C][DirectPieces<DT>::value];
    f32x4 x[2];
};

// Staging of one f32 activation row of k elements (k % 4 == 0, 16-byte
// aligned) in LDS: each of the block's threads carries up to kXStageVec
// 16-byte pieces, so a block of T threads stages rows of up to
// 4 * kXStageVec * T elements, and at most kXStageMaxK (32 KB of LDS).
constexpr int kXStageVec = 8;
constexpr uint32_t kXStageMaxK = 8192;

__host__ __device__ constexpr bool direct_xstage_fits(uint32_t k, uint32_t threads) {
    return k <= kXStageMaxK && (uint64_t)k <= (uint64_t)4 * kXStageVec * threads;
}

struct XStage {
    f32x4 v[kXStageVec];
};

// Piece i of this thread: i * blockDim.x + threadIdx.x, clamped to the last
// piece, so a pass is uniform across the block (threads past the end copy
// the last piece again, writing the value it already has).
__device__ __forceinline__ int xstage_piece(int i, int n4) {
    return min(i * (int)blockDim.x + (int)threadIdx.x, n4 - 1);
}

__device__ __forceinline__ void xstage_issue(const float* xrow, int k, XStage& st) {
    const int n4 = k >> 2;
    const int passes = (n4 + (int)blockDim.x - 1) / (int)blockDim.x;
#pragma unroll
    for (int i = 0; i < kXStageVec; ++i)
        if (i < passes) st.v[i] = reinterpret_cast<const f32x4*>(xrow)[xstage_piece(i, n4)];
}

__device__ __forceinline__ void xstage_store(float* xs, int k, const XStage& st) {
    const int n4 = k >> 2;
    const int passes = (n4 + (int)blockDim.x - 1) / (int)blockDim.x;
#pragma unroll
    for (int i = 0; i < kXStageVec; ++i)
        if (i < passes) reinterpret_cast<f32x4*>(xs)[xstage_piece(i, n4)] = st.v[i];
}

// The same copy by `count` of the block's threads (this one is number
// `idx` among them): piece i * count + idx, clamped to the last piece;
// direct_xstage_fits(k, count) must hold.
__device__ __forceinline__ void xstage_issue_by(const float* xrow, int k, int idx, int count, XStage& st) {
    const int n4 = k >> 2;
    const int passes = (n4 + count - 1) / count;
#pragma unroll
    for (int i = 0; i < kXStageVec; ++i)
        if (i < passes) st.v[i] = reinterpret_cast<const f32x4*>(xrow)[min(i * count + idx, n4 - 1)];
}

__device__ __forceinline__ void xstage_store_by(float* xs, int k, int idx, int count, const XStage& st) {
    const int n4 = k >> 2;
    const int passes = (n4 + count - 1) / count;
#pragma unroll
    for (int i = 0; i < kXStageVec; ++i)
        if (i < passes) reinterpret_cast<f32x4*>(xs)[min(i * count + idx, n4 - 1)] = st.v[i];
}

// Where direct_columns finds the activation row.
enum : int {
    kXFromMemory = 0,  // each slot loads its slice's granule
    kXStageInRing = 1,  // the block stages it in LDS: direct_columns stores the
                        // issued pieces once the weight ring is requested, then
                        // synchronises the block
    kXInLds = 2,        // the caller has staged it and synchronised the block
};

// A wavefront of a staging block that computes no columns still takes its
// part in the copy and the barrier (st: its issued pieces).
__device__ __forceinline__ void xstage_only(int k, float* xs, const XStage& st) {
    xstage_store(xs, k, st);
    __syncthreads();
}

// Columns col0 .. col0+4C-1 of routed row r, whose expert is e (< n_experts);
// the columns from col_end on (col0 < col_end <= n) are not computed: their
// lanes re-read column col0, so every lane issues the same loads.
// On return lane q of slice 0 (lanes 0..3) holds in v[c] the output of
// column col0 + 4c + q (every other lane holds the same totals of its own
// slice group); cvalid[c] says whether that column is one of the computed.
// With XM != kXFromMemory the activation row is the same for the whole
// block, 16-byte aligned with k % 4 == 0 and direct_xstage_fits(k,
// blockDim.x), and xs is LDS for its k floats.  With kXStageInRing every
// wavefront of the block has issued the copy (xstage_issue into *xst) and
// then calls this (or xstage_only): issuing the copy early lets its latency
// hide under the ring's fill.  WHOLE: the caller guarantees 16-byte rows and
// k a multiple of 128, so every round takes the pipelined path.
template <int DT, int C, int D, bool NT, int XM, bool WHOLE = false>
__device__ __forceinline__ void direct_columns(const MatmulArgs& a, uint32_t r, uint32_t e, int col0,
                                               int col_end, float (&v)[C], bool (&cvalid)[C],
                                               float* xs, const XStage* xst) {
    constexpr bool XS = XM != kXFromMemory;
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
    const int full = (WHOLE || a.vec) ? k / kRoundK : 0;

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
        if constexpr (!XS) {
            s.x[0] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK);
            s.x[1] = *reinterpret_cast<const f32x4*>(xlane + g * kRoundK + 4);
        }
    };

    float acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = 0.0f;

    auto consume = [&](int g, const DirectSlot<DT, C>& s) {
        f32x4 x0, x1;
        if constexpr (XS) {
            x0 = *reinterpret_cast<const f32x4*>(xs + g * kRoundK + b * kGranule);
            x1 = *reinterpret_cast<const f32x4*>(xs + g * kRoundK + b * kGranule + 4);
        } else {
            x0 = s.x[0];
            x1 = s.x[1];
        }
        float x[kGranule];
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            x[i] = x0[i];
            x[4 + i] = x1[i];
        }
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c) direct_widen<DT>(s.w[c], w[c]);
#pragma unroll
        for (int i = 0; i < kGranule; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = fma_step(x[i], w[c][i], acc[c]);
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
        if constexpr (XM == kXStageInRing) {
            xstage_store(xs, k, *xst);  // waits for the activation loads only
            __syncthreads();
        }
        int g = 0;
        // steady state: every round refills its slot; the scheduling barrier
        // keeps rounds in order so each wait is only for the oldest slot
        for (; g + 2 * D <= full; g += D) {
#pragma unroll
            for (int d = 0; d < D; ++d) {
                consume(g + d, ring[d]);
                fetch(g + d + D, ring[d]);
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        // the last vector rounds (slots stay in order)
#pragma unroll
        for (int j = 0; j < 2 * D; ++j) {
            const int gg = g + j;
            if (gg < full) {
                consume(gg, ring[j % D]);
                if (gg + D < full) fetch(gg + D, ring[j % D]);
            }
        }
    } else if constexpr (XM == kXStageInRing) {
        xstage_store(xs, k, *xst);
        __syncthreads();
    }
    // rounds that need masked loads (k tail, or rows not 16-byte aligned)
    for (int g = full; !WHOLE && g < rounds; ++g) {
        float x[kGranule];
        load_input_granule(xrow, g * kRoundK + b * kGranule, k, true, false, x);
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c)
            load_weight_granule<DT>(wrow[c] - (size_t)b * kGranule * S, g * kRoundK + b * kGranule, k,
                                    cvalid[c], false, w[c]);
#pragma unroll
        for (int i = 0; i < kGranule; ++i)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[c] = fma_step(x[i], w[c][i], acc[c]);
    }

#pragma unroll
    for (int c = 0; c < C; ++c) v[c] = slice_tree(acc[c]);
}

}  // namespace eidm
