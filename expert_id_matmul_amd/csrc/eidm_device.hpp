// eidm_device.hpp -- device helpers shared by the Direct and Grouped kernels.
//
// Both matmul forms must give identical bits (mlx-native 0.13.0,
// src/ops/dense_matmul_id_auto.rs: the value-independence theorem statement
// says the two routes share input addressing, expert base, weight index,
// widening and the f32 multiply-add, and differ only in which independent
// output rows they compute together).  Here that is enforced by construction:
// every helper below that touches a value is used by both kernels, and both
// accumulate with the same matrix-core instruction in the same order.
//
// The fixed reduction order (the "canonical order") for one output y[r, j]:
//   * k is cut into granules of 8 consecutive elements;
//   * granule g belongs to slice g mod 16 (16 slices);
//   * slice b accumulates, from +0, its products w*x one at a time in
//     ascending k, each step a single-rounding fused multiply-add;
//   * the 16 slice sums are combined pairwise: (b, b^8), then (b, b^4),
//     then (b, b^2), then (b, b^1).
// Elements past k contribute 0*0 steps in both kernels alike.
//
// The accumulation step is a single-rounding f32 fused multiply-add.  The
// Grouped kernel issues it on the matrix core as v_mfma_f32_4x4x1_16b_f32:
// 16 independent 4x4 blocks with one product per output.  Block b of the
// instruction is slice b; in block b, lane 4b+i feeds A-row i and B-column
// i, and output VGPR v of lane 4b+i holds element (row v, column i).  The
// Direct kernels, which need one A-row only, issue the same step on the
// vector ALU as v_fma_f32, lane 4b+i computing element (row 0, column i)
// itself.  On gfx950 the two instructions return the same bits for every
// operand class (normal, subnormal, zero, infinite, NaN with its payload),
// which was measured over 4.2e8 random operand triples; the bitwise
// Direct/Grouped tests check it again on the library's own outputs.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace eidm {

typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kDtypeF32 = 0;
constexpr int kDtypeF16 = 1;
constexpr int kDtypeBF16 = 2;

constexpr int kGranule = 8;                     // k elements per granule
constexpr int kSlices = 16;                     // granules per round = MFMA blocks
constexpr int kRoundK = kGranule * kSlices;     // 128 k elements per round

template <int DT> struct DtypeSize;
template <> struct DtypeSize<kDtypeF32> { static constexpr int value = 4; };
template <> struct DtypeSize<kDtypeF16> { static constexpr int value = 2; };
template <> struct DtypeSize<kDtypeBF16> { static constexpr int value = 2; };

// ---------------------------------------------------------------- widening
// Exact conversion of one native scalar (its raw bits) to f32.
template <int DT> __device__ __forceinline__ float widen_bits(uint32_t bits);
template <> __device__ __forceinline__ float widen_bits<kDtypeF32>(uint32_t bits) {
    return __uint_as_float(bits);
}
template <> __device__ __forceinline__ float widen_bits<kDtypeBF16>(uint32_t bits) {
    return __uint_as_float(bits << 16);
}
template <> __device__ __forceinline__ float widen_bits<kDtypeF16>(uint32_t bits) {
    _Float16 h = __builtin_bit_cast(_Float16, (uint16_t)bits);
    return (float)h;
}

// Widen two packed 16-bit scalars (low half first).
template <int DT> __device__ __forceinline__ void widen_pair(uint32_t packed, float& lo, float& hi);
template <> __device__ __forceinline__ void widen_pair<kDtypeBF16>(uint32_t packed, float& lo, float& hi) {
    lo = __uint_as_float(packed << 16);
    hi = __uint_as_float(packed & 0xffff0000u);
}
template <> __device__ __forceinline__ void widen_pair<kDtypeF16>(uint32_t packed, float& lo, float& hi) {
    lo = widen_bits<kDtypeF16>(packed & 0xffffu);
    hi = widen_bits<kDtypeF16>(packed >> 16);
}

// ---------------------------------------------------------------- loads
// One granule of a weight row: elements kk .. kk+7 of the row starting at
// `row` (byte pointer), widened.  Elements at or past k, and every element
// of an invalid row, read as 0 and touch no memory.  `vec` promises that the
// row start is 16-byte aligned (so a full granule is one or two 16-byte
// loads).
template <int DT>
__device__ __forceinline__ void load_weight_granule(const uint8_t* row, int kk, int k, bool valid,
                                                    bool vec, float (&w)[kGranule]) {
    constexpr int S = DtypeSize<DT>::value;
    if (valid && vec && kk + kGranule <= k) {
        if constexpr (DT == kDtypeF32) {
            const uint4 a = *reinterpret_cast<const uint4*>(row + (size_t)kk * S);
            const uint4 b = *reinterpret_cast<const uint4*>(row + (size_t)kk * S + 16);
            w[0] = __uint_as_float(a.x); w[1] = __uint_as_float(a.y);
            w[2] = __uint_as_float(a.z); w[3] = __uint_as_float(a.w);
            w[4] = __uint_as_float(b.x); w[5] = __uint_as_float(b.y);
            w[6] = __uint_as_float(b.z); w[7] = __uint_as_float(b.w);
        } else {
            const uint4 a = *reinterpret_cast<const uint4*>(row + (size_t)kk * S);
            widen_pair<DT>(a.x, w[0], w[1]);
            widen_pair<DT>(a.y, w[2], w[3]);
            widen_pair<DT>(a.z, w[4], w[5]);
            widen_pair<DT>(a.w, w[6], w[7]);
        }
        return;
    }
#pragma unroll
    for (int i = 0; i < kGranule; ++i) {
        float v = 0.0f;
        if (valid && kk + i < k) {
            uint32_t bits;
            if constexpr (S == 4) {
                bits = *reinterpret_cast<const uint32_t*>(row + (size_t)(kk + i) * 4);
            } else {
                bits = *reinterpret_cast<const uint16_t*>(row + (size_t)(kk + i) * 2);
            }
            v = widen_bits<DT>(bits);
        }
        w[i] = v;
    }
}

// One granule of an f32 activation row (same masking rules).
__device__ __forceinline__ void load_input_granule(const float* row, int kk, int k, bool valid,
                                                   bool vec, float (&x)[kGranule]) {
    if (valid && vec && kk + kGranule <= k) {
        const float4 a = *reinterpret_cast<const float4*>(row + kk);
        const float4 b = *reinterpret_cast<const float4*>(row + kk + 4);
        x[0] = a.x; x[1] = a.y; x[2] = a.z; x[3] = a.w;
        x[4] = b.x; x[5] = b.y; x[6] = b.z; x[7] = b.w;
        return;
    }
#pragma unroll
    for (int i = 0; i < kGranule; ++i) x[i] = (valid && kk + i < k) ? row[kk + i] : 0.0f;
}

// ---------------------------------------------------------------- accumulate
// One canonical accumulation step for all 16 slices at once (matrix core).
__device__ __forceinline__ f32x4 mfma_step(float a, float b, f32x4 acc) {
    return __builtin_amdgcn_mfma_f32_4x4x1f32(a, b, acc, 0, 0, 0);
}

// The same step for this lane's own (slice, column) element (vector ALU).
__device__ __forceinline__ float fma_step(float a, float b, float acc) {
    return __builtin_fmaf(a, b, acc);
}

// Combine the 16 slice sums held by lanes 4b+i (b = 0..15) into the total,
// in the canonical pairing; afterwards every lane 4b+i holds the total of
// column i.  f32 addition is commutative, so both partners of each pair
// compute the same bits.
__device__ __forceinline__ float slice_tree(float v) {
    v += __shfl_xor(v, 32);  // slice b with b^8
    v += __shfl_xor(v, 16);  // b^4
    v += __shfl_xor(v, 8);   // b^2
    v += __shfl_xor(v, 4);   // b^1
    return v;
}

__device__ __forceinline__ float quiet_nan() { return __uint_as_float(0x7fc00000u); }

}  // namespace eidm
