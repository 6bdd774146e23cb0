// noalloc.hip -- the expert-ID matmul for callers that cannot allocate
// device memory: eidm_matmul_id with the Grouped route's id -> row map in a
// fixed device array owned by the library instead of a caller scratch buffer.
//
// The array is a file-scope device variable of kStaticScratchBytes; every
// GPU the library runs on holds its own copy until the process ends.  Its
// address on a device is taken once, with that device current, through
// hipGetSymbolAddress, and kept per device; the kernels receive that
// address.  The map kernels overwrite every word of the map they build, so
// nothing in the array has to start at zero.  All calls on one GPU share the
// array: calls whose work overlaps in time on one GPU (two streams, two host
// threads) race on it.
#include <hip/hip_runtime.h>

#include <mutex>

#include "eidm.h"
#include "eidm_internal.hpp"

namespace {

constexpr uint64_t kStaticScratchBytes = 8ull << 20;  // 8 MiB per device
constexpr int kMaxDevices = 64;

__device__ __align__(256) uint8_t scratch[kStaticScratchBytes];

std::mutex g_mu;
void* g_scratch[kMaxDevices];  // device address of `scratch` per device (null: not taken yet)

// The array's device address on the current device (taken on first use).
int static_scratch(void** out) {
    int dev = -1;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return eidm::api_fail(EIDM_E_DEVICE, "hipGetDevice: %s", hipGetErrorString(err));
    if (dev < 0 || dev >= kMaxDevices)
        return eidm::api_fail(EIDM_E_UNSUPPORTED, "device %d beyond the %d the library tracks", dev, kMaxDevices);
    std::lock_guard<std::mutex> lock(g_mu);
    if (!g_scratch[dev]) {
        void* p = nullptr;
        err = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        if (err != hipSuccess || !p)
            return eidm::api_fail(EIDM_E_DEVICE, "address of the static scratch array on device %d: %s", dev,
                                  hipGetErrorString(err));
        g_scratch[dev] = p;
    }
    *out = g_scratch[dev];
    return EIDM_OK;
}

}  // namespace

extern "C" int eidm_matmul_id_noalloc(const eidm_shape* shape, int route, const void* weights,
                                      uint64_t weight_bytes, const float* input, const uint32_t* ids,
                                      float* output, void* stream, int* route_taken) {
    eidm::ReceiptScope dispatch_receipt;
    eidm_requirements req{};
    req.struct_size = sizeof(req);
    int rc = eidm_query(shape, route == EIDM_ROUTE_AUTO ? EIDM_ROUTE_GROUPED : route, &req);
    if (rc) return rc;
    if (route != EIDM_ROUTE_AUTO && req.scratch_bytes > kStaticScratchBytes)
        return eidm::api_fail(EIDM_E_SIZE,
                              "the route needs %llu bytes of scratch for this shape, above the %llu bytes "
                              "of the library's static array",
                              (unsigned long long)req.scratch_bytes, (unsigned long long)kStaticScratchBytes);
    void* s = nullptr;
    uint64_t sbytes = 0;
    if (route != EIDM_ROUTE_DIRECT || req.scratch_bytes) {
        rc = static_scratch(&s);
        if (rc) return rc;
        sbytes = kStaticScratchBytes;  // AUTO keeps Direct when Grouped's scratch would not fit
    }
    return eidm_matmul_id(shape, route, weights, weight_bytes, input, ids, output, s, sbytes, stream, route_taken);
}
