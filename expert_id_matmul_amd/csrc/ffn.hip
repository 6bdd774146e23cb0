// ffn.hip -- the mixture-of-experts expert FFN over routed rows:
// route -> gate and up projections (shared-layout matmul_id) ->
// h = silu(gate) * up -> down projection (slotted-layout matmul_id over h) ->
// gate-weighted combine.
//
// hf2q, src/inference/models/qwen35/dense_ffn_arena.rs, MoeFfnArena: ids and
// weights are [seq*topk]; gate_all, up_all and h_all are [total_rows, m_moe]
// f32; y_all is [total_rows, h]; the weighted reduce writes [seq, h].
// cortiq-engine 0.7.7, src/mimo_moe.rs, bank_tests: the reference output is
// the sum over picks of w * down(silu(gate.x) (*) up.x).
// hf2q 0.1.1, src/inference/spec_decode/eagle3/forward.rs: the SwiGLU MLP
// applies silu(gate) * up element-wise between the projections.
//
// Each projection is the library's matmul_id (Direct or Grouped, identical
// bits), so the FFN inherits the fixed reduction order; silu(v) is
// v / (1 + exp(-v)) in f32 with the library's correctly rounded division.
#include <hip/hip_runtime.h>

#include "eidm.h"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

// h[i] = silu(g[i]) * u[i], in place over g (16-byte vectors when aligned)
__global__ __launch_bounds__(256) void silu_mul_kernel(float* __restrict__ g, const float* __restrict__ u,
                                                       uint64_t count) {
    const uint64_t quads = count / 4;
    const uint64_t stride = (uint64_t)gridDim.x * blockDim.x;
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < quads; i += stride) {
        float4 a = reinterpret_cast<float4*>(g)[i];
        const float4 b = reinterpret_cast<const float4*>(u)[i];
        a.x = __fdiv_rn(a.x, 1.0f + expf(-a.x)) * b.x;
        a.y = __fdiv_rn(a.y, 1.0f + expf(-a.y)) * b.y;
        a.z = __fdiv_rn(a.z, 1.0f + expf(-a.z)) * b.z;
        a.w = __fdiv_rn(a.w, 1.0f + expf(-a.w)) * b.w;
        reinterpret_cast<float4*>(g)[i] = a;
    }
    for (uint64_t i = quads * 4 + (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count; i += stride)
        g[i] = __fdiv_rn(g[i], 1.0f + expf(-g[i])) * u[i];
}

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

eidm_shape projection(const eidm_ffn_shape* f, bool down) {
    eidm_shape s{};
    s.struct_size = sizeof(eidm_shape);
    s.weight_dtype = f->weight_dtype;
    s.m = f->m;
    s.n = down ? f->hidden : f->inter;
    s.k = down ? f->inter : f->hidden;
    s.top_k = f->top_k;
    s.n_experts = f->n_experts;
    s.expert_stride_bytes = down ? f->down_stride_bytes : f->gate_up_stride_bytes;
    s.input_layout = down ? EIDM_LAYOUT_SLOTTED : EIDM_LAYOUT_SHARED_PER_TOKEN;
    s.id_multiplicity = EIDM_IDS_DISTINCT_PER_TOKEN;
    return s;
}

// scratch: gate/h [R, inter] | up [R, inter] | y [R, hidden] | grouped scratch
struct FfnLayout {
    uint64_t gate, up, y, grouped, total, grouped_bytes;
};

int ffn_layout(const eidm_ffn_shape* f, int route, FfnLayout* l, eidm_shape* gu, eidm_shape* dn) {
    if (!f) return api_fail(EIDM_E_INVALID, "shape is NULL");
    if (f->struct_size != sizeof(eidm_ffn_shape))
        return api_fail(EIDM_E_INVALID, "ffn shape struct_size %u, expected %zu", f->struct_size,
                        sizeof(eidm_ffn_shape));
    *gu = projection(f, false);
    *dn = projection(f, true);
    eidm_requirements rg{}, rd{};
    rg.struct_size = rd.struct_size = sizeof(eidm_requirements);
    int rc = eidm_query(gu, route, &rg);
    if (rc) return rc;
    rc = eidm_query(dn, route, &rd);
    if (rc) return rc;
    uint64_t off = 0;
    l->gate = off;
    off = align256(off + rg.output_elements * 4);
    l->up = off;
    off = align256(off + rg.output_elements * 4);
    l->y = off;
    off = align256(off + rd.output_elements * 4);
    l->grouped = off;
    // Grouped scratch for either projection (same m, top_k, n_experts: the
    // same map sizes); query it on the Grouped route whatever `route` is,
    // so AUTO can take Grouped
    eidm_requirements qg{};
    qg.struct_size = sizeof(qg);
    l->grouped_bytes = eidm_query(gu, EIDM_ROUTE_GROUPED, &qg) == EIDM_OK ? qg.scratch_bytes : 0;
    eidm_requirements qd{};
    qd.struct_size = sizeof(qd);
    if (eidm_query(dn, EIDM_ROUTE_GROUPED, &qd) == EIDM_OK && qd.scratch_bytes > l->grouped_bytes)
        l->grouped_bytes = qd.scratch_bytes;
    l->total = off + l->grouped_bytes;
    return api_ok();
}

}  // namespace
}  // namespace eidm

extern "C" {

uint64_t eidm_moe_ffn_scratch_bytes(const eidm_ffn_shape* shape) {
    eidm::FfnLayout l{};
    eidm_shape gu{}, dn{};
    if (eidm::ffn_layout(shape, EIDM_ROUTE_AUTO, &l, &gu, &dn) != EIDM_OK) return 0;
    return l.total;
}

int eidm_moe_ffn(const eidm_ffn_shape* shape, int route, const void* w_gate, const void* w_up,
                 uint64_t gate_up_bytes, const void* w_down, uint64_t down_bytes, const float* x,
                 const float* logits, const float* bias, int renormalize, uint32_t* ids, float* gates,
                 float* out, void* scratch, uint64_t scratch_bytes, void* stream, int* route_taken) {
    using eidm::api_fail;
    eidm::ReceiptScope dispatch_receipt;
    eidm::FfnLayout l{};
    eidm_shape gu{}, dn{};
    int rc = eidm::ffn_layout(shape, route, &l, &gu, &dn);
    if (rc) return rc;
    if (!w_gate || !w_up || !w_down || !x || !logits || !ids || !gates || !out || !scratch)
        return api_fail(EIDM_E_INVALID, "an FFN buffer is NULL");
    if (scratch_bytes < l.total)
        return api_fail(EIDM_E_SIZE, "the FFN needs %llu bytes of scratch, got %llu", (unsigned long long)l.total,
                        (unsigned long long)scratch_bytes);
    if (reinterpret_cast<uintptr_t>(scratch) % 256)
        return api_fail(EIDM_E_ALIGN, "the FFN scratch must be 256-byte aligned");
    // every check of the five steps, before anything is enqueued
    uint8_t* ws = static_cast<uint8_t*>(scratch);
    float* g = reinterpret_cast<float*>(ws + l.gate);
    float* u = reinterpret_cast<float*>(ws + l.up);
    float* y = reinterpret_cast<float*>(ws + l.y);
    void* grouped = l.grouped_bytes ? ws + l.grouped : nullptr;
    eidm_requirements req{};
    req.struct_size = sizeof(req);
    if ((rc = eidm_query(&gu, route, &req))) return rc;
    if (gate_up_bytes < req.required_weight_bytes)
        return api_fail(EIDM_E_SIZE, "gate/up weights: %llu bytes needed, %llu given",
                        (unsigned long long)req.required_weight_bytes, (unsigned long long)gate_up_bytes);
    eidm_requirements reqd{};
    reqd.struct_size = sizeof(reqd);
    if ((rc = eidm_query(&dn, route, &reqd))) return rc;
    if (down_bytes < reqd.required_weight_bytes)
        return api_fail(EIDM_E_SIZE, "down weights: %llu bytes needed, %llu given",
                        (unsigned long long)reqd.required_weight_bytes, (unsigned long long)down_bytes);
    const int size = shape->weight_dtype == EIDM_DTYPE_F32 ? 4 : 2;
    const uintptr_t wa = reinterpret_cast<uintptr_t>(w_gate) | reinterpret_cast<uintptr_t>(w_up) |
                         reinterpret_cast<uintptr_t>(w_down);
    if (wa % size) return api_fail(EIDM_E_ALIGN, "weights must be aligned to the scalar size");
    if ((reinterpret_cast<uintptr_t>(x) | reinterpret_cast<uintptr_t>(logits) | reinterpret_cast<uintptr_t>(ids) |
         reinterpret_cast<uintptr_t>(gates) | reinterpret_cast<uintptr_t>(out) |
         reinterpret_cast<uintptr_t>(bias)) % 4)
        return api_fail(EIDM_E_ALIGN, "FFN buffers must be 4-byte aligned");
    if (shape->top_k > eidm::kMaxRouterTopK || shape->n_experts > eidm::kMaxExperts ||
        shape->top_k > shape->n_experts)
        return api_fail(EIDM_E_UNSUPPORTED, "router limits: top_k <= min(n_experts, %u), n_experts <= %u",
                        eidm::kMaxRouterTopK, eidm::kMaxExperts);

    rc = eidm_route_topk(logits, bias, shape->m, shape->n_experts, shape->top_k, renormalize, ids, gates, stream);
    if (rc) return rc;
    // the three projections share the ids, routed rows and experts: the
    // first Grouped one builds the id -> row map in the scratch, the others
    // reuse it
    hipStream_t st = static_cast<hipStream_t>(stream);
    bool map_ready = false;
    int taken = 0;
    rc = eidm::matmul_id_shared_map(&gu, route, w_gate, gate_up_bytes, x, ids, g, grouped, l.grouped_bytes, st,
                                    &map_ready, &taken);
    if (rc) return rc;
    rc = eidm::matmul_id_shared_map(&gu, route, w_up, gate_up_bytes, x, ids, u, grouped, l.grouped_bytes, st,
                                    &map_ready, nullptr);
    if (rc) return rc;
    const uint64_t count = (uint64_t)shape->m * shape->top_k * shape->inter;
    uint64_t blocks = (count / 4 + 255) / 256;
    if (blocks == 0) blocks = 1;
    if (blocks > 65536) blocks = 65536;
    hipLaunchKernelGGL(eidm::silu_mul_kernel, dim3((uint32_t)blocks), dim3(256), 0,
                       static_cast<hipStream_t>(stream), g, u, count);
    const hipError_t err = eidm::launched(EIDM_KERNEL_SILU_MUL, (uint32_t)blocks, 256, 0);
    if (err != hipSuccess) return api_fail(EIDM_E_DEVICE, "silu * up launch: %s", hipGetErrorString(err));
    rc = eidm::matmul_id_shared_map(&dn, route, w_down, down_bytes, g, ids, y, grouped, l.grouped_bytes, st,
                                    &map_ready, nullptr);
    if (rc) return rc;
    rc = eidm_combine(shape->m, shape->top_k, shape->hidden, y, gates, out, stream);
    if (rc) return rc;
    eidm::receipt_route(taken);
    if (route_taken) *route_taken = taken;
    return eidm::api_ok();
}

}  // extern "C"
