// validate.hip -- device-side check of a routed id table: every id names an
// expert, and (for distinct-per-token tables) no token repeats one.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: the shape key carries
// the id multiplicity (DenseMatmulIdMultiplicity) and the calibration's
// profile ids are distinct per token unless the repeating profile asks
// otherwise (fn calibration_buffers); the page does not say what happens to
// an id outside [0, n_experts), so this check makes such a table an error
// the caller can see before any matmul runs.
//
// One thread per routed entry r = t*top_k + s; an entry is bad when its id is
// >= n_experts or, for distinct tables, equals an earlier slot of its token.
// The smallest bad r is kept with an atomic minimum in a per-device word.
#include <hip/hip_runtime.h>

#include <climits>

#include "eidm_internal.hpp"

namespace eidm {
namespace {

__device__ int g_first_bad;  // one per device (module global)

__global__ __launch_bounds__(256) void validate_kernel(const uint32_t* __restrict__ ids, uint32_t m,
                                                       uint32_t top_k, uint32_t n_experts, int distinct) {
    const uint64_t total = (uint64_t)m * top_k;
    for (uint64_t r = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; r < total;
         r += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t id = ids[r];
        bool bad = id >= n_experts;
        if (!bad && distinct) {
            const uint64_t first = r - r % top_k;
            for (uint64_t p = first; p < r; ++p)
                if (ids[p] == id) {
                    bad = true;
                    break;
                }
        }
        if (bad) atomicMin(&g_first_bad, (int)r);
    }
}

}  // namespace

hipError_t run_validate(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts, int distinct,
                        hipStream_t stream, int* first_bad) {
    const int none = INT_MAX;
    hipError_t err = hipMemcpyToSymbolAsync(HIP_SYMBOL(g_first_bad), &none, sizeof(int), 0,
                                            hipMemcpyHostToDevice, stream);
    if (err != hipSuccess) return err;
    const uint64_t total = (uint64_t)m * top_k;
    uint64_t blocks = (total + 255) / 256;
    if (blocks > 4096) blocks = 4096;
    hipLaunchKernelGGL(validate_kernel, dim3((uint32_t)blocks), dim3(256), 0, stream, ids, m, top_k,
                       n_experts, distinct);
    err = launched(EIDM_KERNEL_VALIDATE, (uint32_t)blocks, 256, 0);
    if (err != hipSuccess) return err;
    int result = none;
    err = hipMemcpyFromSymbolAsync(&result, HIP_SYMBOL(g_first_bad), sizeof(int), 0,
                                   hipMemcpyDeviceToHost, stream);
    if (err != hipSuccess) return err;
    err = hipStreamSynchronize(stream);
    if (err != hipSuccess) return err;
    *first_bad = result == none ? -1 : result;
    return hipSuccess;
}

}  // namespace eidm
