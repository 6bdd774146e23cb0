// eidm_internal.hpp -- kernel launchers behind the C ABI (host side).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "eidm.h"

namespace eidm {

// Largest expert count the kernels take (router state per lane, map tables).
constexpr uint32_t kMaxExperts = 2048;

// Largest top_k the router takes (one pick per lane).
constexpr uint32_t kMaxRouterTopK = 64;
// fused route -> Direct -> combine: one wavefront per slot in a block
constexpr uint32_t kMaxMoeDirectTopK = 16;

struct MatmulArgs {
    int dtype;
    uint32_t m, n, k, top_k, n_experts;
    uint64_t stride;
    int layout;                 // 0 shared per token, 1 slotted
    const void* weights;
    const float* input;
    const uint32_t* ids;
    float* output;
    bool vec;                   // 16-byte aligned rows: vector loads allowed
    int arith;                  // eidm_arith
    uint16_t* xsplit;           // SPLIT16: the split activations (scratch), else null
};

// Device pointers into a Grouped scratch buffer.
struct MapBuffers {
    uint32_t* hist;     // [blocks][n_experts+1]
    uint32_t* counts;   // [n_experts+1]
    uint32_t* offsets;  // [n_experts+2]
    uint32_t* rows;     // [m*top_k]
};

uint32_t map_waves(uint32_t n_experts);
uint32_t map_blocks(uint64_t routed_rows, uint32_t n_experts);
uint64_t map_hist_elements(uint64_t routed_rows, uint32_t n_experts);

// error state of the C ABI (thread-local message; see eidm_last_error)
int api_fail(int code, const char* fmt, ...);
int api_ok();

// The dispatch receipt (see eidm_last_dispatch): each public entry point
// starts a new one on the calling thread; every kernel launch is noted.
// The outermost scope on a thread starts the receipt; nested entry points
// (a library call made by another one) add to it.
struct ReceiptScope {
    ReceiptScope();
    ~ReceiptScope();
    ReceiptScope(const ReceiptScope&) = delete;
    ReceiptScope& operator=(const ReceiptScope&) = delete;
};
void receipt_route(int route);
void note_launch(int kernel, uint32_t grid, uint32_t block, uint32_t lds_bytes);
// hipGetLastError() after a launch; the launch goes on the receipt only when
// it was accepted.
hipError_t launched(int kernel, uint32_t grid, uint32_t block, uint32_t lds_bytes);

hipError_t launch_route(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                        uint32_t top_k, int renormalize, uint32_t* ids, float* gates,
                        hipStream_t stream);
hipError_t launch_map(const uint32_t* ids, uint32_t routed_rows, uint32_t n_experts,
                      const MapBuffers& buf, hipStream_t stream);
// eidm_matmul_id for a sequence of calls over one set of ids (and one
// scratch): a Grouped call skips the id -> row map when *map_ready says an
// earlier Grouped call of the sequence left it in the scratch, and sets
// *map_ready when it builds it.
int matmul_id_shared_map(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                         const float* input, const uint32_t* ids, float* output, void* scratch,
                         uint64_t scratch_bytes, hipStream_t stream, bool* map_ready, int* route_taken);
hipError_t launch_direct(const MatmulArgs& a, hipStream_t stream);
hipError_t launch_grouped(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                          hipStream_t stream);
// The Grouped kernel on the 16x16x1 matrix-core step (16-bit weights, vector
// rows, at least two rounds, 32-bit offsets); launch_grouped picks it when
// grouped16_supported says so.
bool grouped16_supported(const MatmulArgs& a);
hipError_t launch_grouped16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream);
// jobs of at most this many rounds of k run the build of the same kernel
// that keeps its accumulators in the accumulation registers
#ifndef EIDM_G16_ACC_ROUNDS
#define EIDM_G16_ACC_ROUNDS 12
#endif
constexpr uint32_t kG16AccRounds = EIDM_G16_ACC_ROUNDS;
hipError_t launch_grouped16_acc(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream);
// The split-16 arithmetic: the activation split (input -> a.xsplit), then
// the Direct or the Grouped form.
// bytes of the split activations of in_rows rows of k elements
uint64_t split16_bytes(uint64_t in_rows, uint32_t k);
hipError_t launch_split16_x(const MatmulArgs& a, hipStream_t stream);
// the id -> row map (one-launch form) and the activation split in one launch,
// when the map fits that form
bool map_split16_x_fits(const MatmulArgs& a);
hipError_t launch_map_split16_x(const MatmulArgs& a, const MapBuffers& buf, hipStream_t stream);
hipError_t launch_direct_split16(const MatmulArgs& a, hipStream_t stream);
hipError_t launch_grouped_split16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream);
hipError_t launch_combine(uint32_t m, uint32_t top_k, uint32_t n, const float* y,
                          const float* gates, float* out, hipStream_t stream);
bool moe_direct_supported(uint32_t top_k, uint32_t n_experts);
// synchronous: waits for `stream`; *first_bad = smallest bad routed index or -1
hipError_t run_validate(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts, int distinct,
                        hipStream_t stream, int* first_bad);
// a.ids is ignored: the kernel writes the picks to `ids` and reads them itself
hipError_t launch_moe_direct(const MatmulArgs& a, const float* logits, const float* bias, int renormalize,
                             uint32_t* ids, float* gates, float* out, int device_cus, hipStream_t stream);

}  // namespace eidm
