// matmul_direct.hip -- Direct form of the expert-ID matmul: each wavefront
// computes 4*C output columns of one routed row (direct_wave.hpp), streaming
// that expert's weight rows from HBM once.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: fn expected_dispatches
// gives the Direct route one dispatch over (column groups) x (m*top_k routed
// rows); the value-independence theorem statement fixes what it shares with
// the grouped route.  Here a block is WAVES wavefronts of 4*C columns of one
// routed row.
#include "direct_wave.hpp"

#ifndef EIDM_DIRECT_C
#define EIDM_DIRECT_C 2
#endif
#ifndef EIDM_DIRECT_WAVES
#define EIDM_DIRECT_WAVES 2
#endif
#ifndef EIDM_DIRECT_DEPTH
#define EIDM_DIRECT_DEPTH 8
#endif
#ifndef EIDM_DIRECT_NT
#define EIDM_DIRECT_NT 1
#endif

namespace eidm {
namespace {

template <int DT, int C, int WAVES, int D, bool XS>
__global__ __launch_bounds__(64 * WAVES) void direct_kernel(MatmulArgs a) {
    extern __shared__ __align__(16) float xs[];  // the activation row (XS)
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int n = (int)a.n;
    const uint32_t col_blocks = (a.n + 4 * C * WAVES - 1) / (4 * C * WAVES);
    const uint32_t r = blockIdx.x / col_blocks;  // one routed row per block
    const int col0 = ((int)(blockIdx.x % col_blocks) * WAVES + wave) * (4 * C);
    float* yrow = a.output + (size_t)r * a.n;

    const uint32_t e = a.ids[r];
    if (e >= a.n_experts) {  // no weights for this row: quiet NaN (the whole block leaves)
        if (lane < 4 * C && col0 + lane < n) yrow[col0 + lane] = quiet_nan();
        return;
    }
    XStage xst;
    if constexpr (XS) {
        const uint32_t xr = a.layout == 1 ? r : r / a.top_k;
        xstage_issue(a.input + (size_t)xr * a.k, (int)a.k, xst);
        __builtin_amdgcn_sched_barrier(0);  // the activation loads go out before the weights
    }
    if (col0 >= n) {  // wave-uniform
        if constexpr (XS) xstage_only((int)a.k, xs, xst);
        return;
    }
    float v[C];
    bool cvalid[C];
    direct_columns<DT, C, D, EIDM_DIRECT_NT != 0, XS ? kXStageInRing : kXFromMemory>(a, r, e, col0, n, v, cvalid,
                                                                                      xs, &xst);
#pragma unroll
    for (int c = 0; c < C; ++c)
        if (b == 0 && cvalid[c]) yrow[col0 + 4 * c + q] = v[c];
}

// The activation row goes through LDS when the block can stage it in one
// pass; a block is one routed row, so its wavefronts share that row.
template <int DT, int C, int WAVES, int D>
hipError_t launch_cfg(const MatmulArgs& a, hipStream_t stream) {
    const uint32_t cols_per_block = 4 * C * WAVES;
    const dim3 grid(((a.n + cols_per_block - 1) / cols_per_block) * (a.m * a.top_k));
    const bool xs = a.vec && direct_xstage_fits(a.k, 64 * WAVES);
    if (xs)
        hipLaunchKernelGGL((direct_kernel<DT, C, WAVES, D, true>), grid, dim3(64 * WAVES), (size_t)a.k * 4, stream, a);
    else
        hipLaunchKernelGGL((direct_kernel<DT, C, WAVES, D, false>), grid, dim3(64 * WAVES), 0, stream, a);
    return launched(EIDM_KERNEL_DIRECT, grid.x, 64 * WAVES, xs ? a.k * 4 : 0);
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
