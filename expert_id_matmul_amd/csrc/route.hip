// route.hip -- the router kernel: one wavefront per token (route_wave.hpp
// holds the selection and its citation).
#include "eidm_device.hpp"
#include "eidm_internal.hpp"
#include "route_wave.hpp"

namespace eidm {
namespace {

template <int NV>
__global__ __launch_bounds__(256) void route_kernel(const float* __restrict__ logits,
                                                    const float* __restrict__ bias, uint32_t m,
                                                    uint32_t n_experts, uint32_t top_k,
                                                    int renormalize, uint32_t* __restrict__ ids,
                                                    float* __restrict__ gates) {
    const int lane = threadIdx.x & 63;
    const uint32_t t = blockIdx.x * 4 + (threadIdx.x >> 6);
    if (t >= m) return;
    uint32_t id;
    float gate;
    route_token<NV>(logits + (size_t)t * n_experts, bias, n_experts, top_k, renormalize, id, gate);
    if (lane < (int)top_k) {
        ids[(size_t)t * top_k + lane] = id;
        if (gates) gates[(size_t)t * top_k + lane] = gate;
    }
}

template <int NV>
hipError_t launch_nv(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                     uint32_t top_k, int renormalize, uint32_t* ids, float* gates,
                     hipStream_t stream) {
    const dim3 grid((m + 3) / 4);
    hipLaunchKernelGGL(route_kernel<NV>, grid, dim3(256), 0, stream, logits, bias, m, n_experts,
                       top_k, renormalize, ids, gates);
    return launched(EIDM_KERNEL_ROUTE, grid.x, 256, 0);
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
