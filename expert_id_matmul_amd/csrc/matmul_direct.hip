// matmul_direct.hip -- Direct form of the expert-ID matmul: each wavefront
// computes 4*C output columns of one routed row, streaming that expert's
// weight rows from HBM once.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: fn expected_dispatches
// gives the Direct route one dispatch over (column groups) x (m*top_k routed
// rows), with no threadgroup memory; the value-independence theorem statement
// fixes what it shares with the grouped route.  Here the column group is
// 4*C columns per wavefront and WAVES wavefronts per block.
//
// Per round (128 k), lane 4b+q (slice b, column q) loads one 8-element
// granule of weight row col0+4c+q for each c, the lanes with q == 0 load the
// activation granule (the only valid A-row of the matrix-core block), and
// 8*C accumulation steps follow.  Weights are read with 16-byte loads that
// cover 256 contiguous bytes per row per round.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

template <int DT, int C, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void direct_kernel(MatmulArgs a) {
    constexpr int S = DtypeSize<DT>::value;
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int n = (int)a.n, k = (int)a.k;
    const uint32_t col_blocks = (a.n + 4 * C * WAVES - 1) / (4 * C * WAVES);
    const uint32_t r = blockIdx.x / col_blocks;
    const int col0 = ((int)(blockIdx.x % col_blocks) * WAVES + wave) * (4 * C);
    if (col0 >= n) return;
    float* yrow = a.output + (size_t)r * a.n;

    const uint32_t e = a.ids[r];
    if (e >= a.n_experts) {  // no weights for this row: quiet NaN, read nothing
        if (lane < 4 * C && col0 + lane < n) yrow[col0 + lane] = quiet_nan();
        return;
    }
    const uint32_t xr = a.layout == 1 ? r : r / a.top_k;
    const float* xrow = a.input + (size_t)xr * a.k;
    const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;

    const uint8_t* wrow[C];
    bool cvalid[C];
#pragma unroll
    for (int c = 0; c < C; ++c) {
        const int col = col0 + 4 * c + q;
        cvalid[c] = col < n;
        wrow[c] = wexp + (size_t)(cvalid[c] ? col : 0) * a.k * S;
    }

    f32x4 acc[C];
#pragma unroll
    for (int c = 0; c < C; ++c) acc[c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    const int rounds = (k + kRoundK - 1) / kRoundK;
    const bool vec = a.vec;
    for (int g = 0; g < rounds; ++g) {
        const int kk = g * kRoundK + b * kGranule;
        float x[kGranule];
        load_input_granule(xrow, kk, k, q == 0, vec, x);
        float w[C][kGranule];
#pragma unroll
        for (int c = 0; c < C; ++c) load_weight_granule<DT>(wrow[c], kk, k, cvalid[c], vec, w[c]);
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

template <int DT, int C, int WAVES>
hipError_t launch_cfg(const MatmulArgs& a, hipStream_t stream) {
    const uint32_t cols_per_block = 4 * C * WAVES;
    const dim3 grid(((a.n + cols_per_block - 1) / cols_per_block) * (a.m * a.top_k));
    hipLaunchKernelGGL((direct_kernel<DT, C, WAVES>), grid, dim3(64 * WAVES), 0, stream, a);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const MatmulArgs& a, hipStream_t stream) {
    return launch_cfg<DT, 1, 4>(a, stream);
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
