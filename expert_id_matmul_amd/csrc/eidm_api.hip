// eidm_api.hip -- the C ABI (include/eidm.h): host-side validation, route
// choice and kernel launches.  Nothing here allocates device memory; every
// check runs before the first launch, so a failed call enqueues nothing.
//
// Validation follows mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs:
// sizes are overflow-checked products (fn checked_product), the weight
// extent must reach the required bytes and the weight pointer must be
// aligned to its scalar size (fn validate_cases), and errors fail closed
// with a message.
#include <hip/hip_runtime.h>

#include <atomic>
#include <mutex>
#include <cstdarg>
#include <cstdio>
#include <cstring>
#include <string>

#include "eidm.h"
#include "eidm_internal.hpp"

namespace {
thread_local std::string g_error;
thread_local eidm_dispatch g_receipt;
thread_local int g_receipt_depth = 0;
}  // namespace

namespace eidm {

ReceiptScope::ReceiptScope() {
    if (g_receipt_depth++ == 0) {
        g_receipt = eidm_dispatch{};
        g_receipt.struct_size = sizeof(eidm_dispatch);
    }
}

ReceiptScope::~ReceiptScope() { --g_receipt_depth; }

void receipt_route(int route) { g_receipt.route = route; }

void note_launch(int kernel, uint32_t grid, uint32_t block, uint32_t lds_bytes) {
    if (g_receipt.recorded < EIDM_MAX_RECORDED_LAUNCHES) {
        eidm_launch& l = g_receipt.launches[g_receipt.recorded++];
        l.kernel = kernel;
        l.grid = grid;
        l.block = block;
        l.lds_bytes = lds_bytes;
    }
    ++g_receipt.dispatch_count;
}

hipError_t launched(int kernel, uint32_t grid, uint32_t block, uint32_t lds_bytes) {
    const hipError_t err = hipGetLastError();
    if (err == hipSuccess) note_launch(kernel, grid, block, lds_bytes);
    return err;
}

int api_fail(int code, const char* fmt, ...) {
    char buf[512];
    va_list ap;
    va_start(ap, fmt);
    vsnprintf(buf, sizeof(buf), fmt, ap);
    va_end(ap);
    g_error = buf;
    return code;
}

int api_ok() {
    g_error.clear();
    return EIDM_OK;
}

}  // namespace eidm

namespace {

using eidm::api_fail;
int ok() { return eidm::api_ok(); }

bool mul_ok(uint64_t a, uint64_t b, uint64_t* out) {
    return !__builtin_mul_overflow(a, b, out);
}

bool add_ok(uint64_t a, uint64_t b, uint64_t* out) {
    return !__builtin_add_overflow(a, b, out);
}

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

int dtype_size(int dtype) {
    switch (dtype) {
    case EIDM_DTYPE_F32: return 4;
    case EIDM_DTYPE_F16: return 2;
    case EIDM_DTYPE_BF16: return 2;
    default: return 0;
    }
}

constexpr uint64_t kIndexLimit = 0x7fffffffull;  // kernels index rows and grids in 31 bits

struct Plan {
    uint64_t routed = 0;
    uint64_t input_elements = 0;
    uint64_t output_elements = 0;
    uint64_t required_weight_bytes = 0;
    uint64_t grouped_scratch = 0;
    uint64_t direct_scratch = 0;  // the split activations (SPLIT16), else 0
    // byte offsets of the grouped scratch sections (the split activations
    // follow the map; a Direct scratch holds them at offset 0)
    uint64_t off_hist = 0, off_counts = 0, off_offsets = 0, off_rows = 0, off_split = 0;
};

int check_shape(const eidm_shape* s, Plan* p) {
    if (!s) return api_fail(EIDM_E_INVALID, "shape is NULL");
    if (s->struct_size != sizeof(eidm_shape))
        return api_fail(EIDM_E_INVALID, "shape.struct_size is %u, expected %zu", s->struct_size,
                    sizeof(eidm_shape));
    const int size = dtype_size(s->weight_dtype);
    if (!size) return api_fail(EIDM_E_INVALID, "unknown weight dtype %d", s->weight_dtype);
    if (s->input_layout != EIDM_LAYOUT_SHARED_PER_TOKEN && s->input_layout != EIDM_LAYOUT_SLOTTED)
        return api_fail(EIDM_E_INVALID, "unknown input layout %d", s->input_layout);
    if (s->id_multiplicity != EIDM_IDS_DISTINCT_PER_TOKEN && s->id_multiplicity != EIDM_IDS_MAY_REPEAT)
        return api_fail(EIDM_E_INVALID, "unknown id multiplicity %d", s->id_multiplicity);
    if (s->arith != EIDM_ARITH_F32 && s->arith != EIDM_ARITH_SPLIT16)
        return api_fail(EIDM_E_INVALID, "unknown arith %d", s->arith);
    if (s->arith == EIDM_ARITH_SPLIT16 && size != 2)
        return api_fail(EIDM_E_UNSUPPORTED, "the split-16 arithmetic needs 16-bit weights");
    if (s->arith == EIDM_ARITH_SPLIT16 && s->k % 8 != 0)
        return api_fail(EIDM_E_UNSUPPORTED, "the split-16 arithmetic needs k a multiple of 8 (k=%u)", s->k);
    if (!s->m || !s->n || !s->k || !s->top_k || !s->n_experts)
        return api_fail(EIDM_E_INVALID, "zero dimension (m=%u n=%u k=%u top_k=%u n_experts=%u)", s->m,
                    s->n, s->k, s->top_k, s->n_experts);
    if (s->n_experts > eidm::kMaxExperts)
        return api_fail(EIDM_E_UNSUPPORTED, "n_experts %u above the supported %u", s->n_experts,
                    eidm::kMaxExperts);
    if (s->id_multiplicity == EIDM_IDS_DISTINCT_PER_TOKEN && s->top_k > s->n_experts)
        return api_fail(EIDM_E_INVALID, "top_k %u distinct ids from %u experts", s->top_k, s->n_experts);
    if (s->n > kIndexLimit || s->k > kIndexLimit)
        return api_fail(EIDM_E_UNSUPPORTED, "n or k at or above 2^31");

    uint64_t body;
    if (!mul_ok((uint64_t)s->n, s->k, &body) || !mul_ok(body, size, &body))
        return api_fail(EIDM_E_INVALID, "expert size overflows");
    if (s->expert_stride_bytes % size)
        return api_fail(EIDM_E_ALIGN, "expert stride %llu is not a multiple of the dtype size %d",
                    (unsigned long long)s->expert_stride_bytes, size);
    if (s->expert_stride_bytes < body)
        return api_fail(EIDM_E_INVALID, "expert stride %llu is shorter than one expert (%llu bytes)",
                    (unsigned long long)s->expert_stride_bytes, (unsigned long long)body);
    uint64_t req;
    if (!mul_ok((uint64_t)(s->n_experts - 1), s->expert_stride_bytes, &req) || !add_ok(req, body, &req))
        return api_fail(EIDM_E_INVALID, "required weight bytes overflow");

    uint64_t routed, in_rows, in_el, out_el;
    if (!mul_ok(s->m, s->top_k, &routed)) return api_fail(EIDM_E_INVALID, "m*top_k overflows");
    if (routed > kIndexLimit) return api_fail(EIDM_E_UNSUPPORTED, "m*top_k at or above 2^31");
    in_rows = s->input_layout == EIDM_LAYOUT_SLOTTED ? routed : s->m;
    if (!mul_ok(in_rows, s->k, &in_el)) return api_fail(EIDM_E_INVALID, "input size overflows");
    if (!mul_ok(routed, s->n, &out_el)) return api_fail(EIDM_E_INVALID, "output size overflows");
    uint64_t direct_blocks;
    if (!mul_ok((s->n + 15) / 16, routed, &direct_blocks) || direct_blocks > kIndexLimit)
        return api_fail(EIDM_E_UNSUPPORTED, "Direct grid of %llu blocks is too large",
                    (unsigned long long)direct_blocks);

    p->routed = routed;
    p->input_elements = in_el;
    p->output_elements = out_el;
    p->required_weight_bytes = req;
    p->off_hist = 0;
    p->off_counts = align256(eidm::map_hist_elements(routed, s->n_experts) * 4);
    p->off_offsets = p->off_counts + align256((uint64_t)(s->n_experts + 1) * 4);
    p->off_rows = p->off_offsets + align256((uint64_t)(s->n_experts + 2) * 4);
    // the row list keeps 32 spare entries: a Grouped kernel reads a job's
    // 32 entries at once, also for the last bucket
    p->off_split = p->off_rows + align256((routed + 32) * 4);
    p->grouped_scratch = p->off_split;
    if (s->arith == EIDM_ARITH_SPLIT16) {
        // three 16-bit parts per input element, rows padded to whole 128-k
        // rounds (16 chunks of 8), plus a 256-byte zero block
        uint64_t split;
        const uint64_t row_chunks = ((uint64_t)s->k + 127) / 128 * 16;
        if (!mul_ok(in_rows, row_chunks, &split) || !mul_ok(split, 48, &split) || !add_ok(split, 256 + 255, &split))
            return api_fail(EIDM_E_INVALID, "split input size overflows");
        p->direct_scratch = split & ~uint64_t(255);
        if (p->direct_scratch < eidm::split16_bytes(in_rows, s->k))
            return api_fail(EIDM_E_INVALID, "split input size mismatch");
        // the split-16 kernels address an expert's matrix and the split
        // activations with 32-bit buffer offsets
        if (body >= (1ull << 31) || p->direct_scratch >= (1ull << 31))
            return api_fail(EIDM_E_UNSUPPORTED,
                            "the split-16 arithmetic needs each expert's matrix and the split activations "
                            "below 2 GiB");
        if (!add_ok(p->grouped_scratch, p->direct_scratch, &p->grouped_scratch))
            return api_fail(EIDM_E_INVALID, "scratch size overflows");
    }
    return EIDM_OK;
}

int resolve_route(const eidm_shape* s, const Plan& p, int route, bool scratch_given,
                  uint64_t scratch_bytes, int* out) {
    switch (route) {
    case EIDM_ROUTE_DIRECT:
        *out = EIDM_ROUTE_DIRECT;
        return EIDM_OK;
    case EIDM_ROUTE_GROUPED:
        *out = EIDM_ROUTE_GROUPED;
        return EIDM_OK;
    case EIDM_ROUTE_AUTO: {
        const bool dense_enough = p.routed >= 2ull * s->n_experts;
        const bool have = !scratch_given || scratch_bytes >= p.grouped_scratch;
        *out = dense_enough && have ? EIDM_ROUTE_GROUPED : EIDM_ROUTE_DIRECT;
        return EIDM_OK;
    }
    default:
        return api_fail(EIDM_E_INVALID, "unknown route %d", route);
    }
}

bool aligned(const void* ptr, uintptr_t a) { return (reinterpret_cast<uintptr_t>(ptr) % a) == 0; }

std::atomic<int> g_cus[64];

int device_cus() {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= 64) return 256;
    int v = g_cus[dev].load(std::memory_order_relaxed);
    if (v > 0) return v;
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || cus <= 0)
        cus = 256;
    g_cus[dev].store(cus, std::memory_order_relaxed);
    return cus;
}

int device_fail(hipError_t err, const char* what) {
    return api_fail(EIDM_E_DEVICE, "%s: %s", what, hipGetErrorString(err));
}

// Validate everything a matmul call needs; fills args, map buffers and route.
int prepare_matmul(const eidm_shape* s, int route, const void* weights, uint64_t weight_bytes,
                   const float* input, const uint32_t* ids, float* output, void* scratch,
                   uint64_t scratch_bytes, eidm::MatmulArgs* args, eidm::MapBuffers* buf,
                   int* chosen) {
    Plan p;
    int rc = check_shape(s, &p);
    if (rc) return rc;
    const int size = dtype_size(s->weight_dtype);
    if (!weights) return api_fail(EIDM_E_INVALID, "weights is NULL");
    if (!aligned(weights, size)) return api_fail(EIDM_E_ALIGN, "weights not aligned to %d bytes", size);
    if (weight_bytes < p.required_weight_bytes)
        return api_fail(EIDM_E_SIZE, "weight extent %llu below the required %llu bytes",
                    (unsigned long long)weight_bytes, (unsigned long long)p.required_weight_bytes);
    if (!input || !ids || !output) return api_fail(EIDM_E_INVALID, "input, ids or output is NULL");
    if (!aligned(input, 4) || !aligned(ids, 4) || !aligned(output, 4))
        return api_fail(EIDM_E_ALIGN, "input, ids and output must be 4-byte aligned");
    const bool split = s->arith == EIDM_ARITH_SPLIT16;
    if (split && (!aligned(weights, 16) || s->expert_stride_bytes % 16 || !aligned(input, 16)))
        return api_fail(EIDM_E_ALIGN, "the split-16 arithmetic needs weights, expert stride and input 16-byte aligned");
    rc = resolve_route(s, p, route, true, scratch ? scratch_bytes : 0, chosen);
    if (rc) return rc;
    args->xsplit = nullptr;
    if (split && *chosen == EIDM_ROUTE_DIRECT) {
        if (!scratch || scratch_bytes < p.direct_scratch)
            return api_fail(EIDM_E_SIZE, "the split-16 Direct route needs %llu bytes of scratch, got %llu",
                            (unsigned long long)p.direct_scratch, (unsigned long long)(scratch ? scratch_bytes : 0));
        if (!aligned(scratch, 256)) return api_fail(EIDM_E_ALIGN, "scratch must be 256-byte aligned");
        args->xsplit = static_cast<uint16_t*>(scratch);
    }
    if (*chosen == EIDM_ROUTE_GROUPED) {
        if (!scratch) return api_fail(EIDM_E_SIZE, "Grouped route needs %llu bytes of scratch, got none",
                                  (unsigned long long)p.grouped_scratch);
        if (scratch_bytes < p.grouped_scratch)
            return api_fail(EIDM_E_SIZE, "Grouped route needs %llu bytes of scratch, got %llu",
                        (unsigned long long)p.grouped_scratch, (unsigned long long)scratch_bytes);
        if (!aligned(scratch, 256)) return api_fail(EIDM_E_ALIGN, "scratch must be 256-byte aligned");
        uint8_t* base = static_cast<uint8_t*>(scratch);
        buf->hist = reinterpret_cast<uint32_t*>(base + p.off_hist);
        buf->counts = reinterpret_cast<uint32_t*>(base + p.off_counts);
        buf->offsets = reinterpret_cast<uint32_t*>(base + p.off_offsets);
        buf->rows = reinterpret_cast<uint32_t*>(base + p.off_rows);
        if (split) args->xsplit = reinterpret_cast<uint16_t*>(base + p.off_split);
    }
    args->dtype = s->weight_dtype;
    args->m = s->m;
    args->n = s->n;
    args->k = s->k;
    args->top_k = s->top_k;
    args->n_experts = s->n_experts;
    args->stride = s->expert_stride_bytes;
    args->layout = s->input_layout;
    args->weights = weights;
    args->input = input;
    args->ids = ids;
    args->output = output;
    args->arith = s->arith;
    args->vec = aligned(weights, 16) && s->expert_stride_bytes % 16 == 0 &&
                ((uint64_t)s->k * size) % 16 == 0 && aligned(input, 16) && s->k % 4 == 0;
    return EIDM_OK;
}

// build_map = false: the id -> row map is already in buf (Grouped only)
int run_matmul(const eidm::MatmulArgs& args, const eidm::MapBuffers& buf, int chosen,
               hipStream_t stream, bool build_map = true) {
    hipError_t err;
    if (args.arith == EIDM_ARITH_SPLIT16) {
        if (chosen == EIDM_ROUTE_GROUPED && build_map && eidm::map_split16_x_fits(args)) {
            // the map and the activation split side by side in one launch
            err = eidm::launch_map_split16_x(args, buf, stream);
            if (err != hipSuccess) return device_fail(err, "map and activation split launch");
        } else {
            err = eidm::launch_split16_x(args, stream);
            if (err != hipSuccess) return device_fail(err, "activation split launch");
            if (chosen == EIDM_ROUTE_GROUPED && build_map) {
                err = eidm::launch_map(args.ids, args.m * args.top_k, args.n_experts, buf, stream);
                if (err != hipSuccess) return device_fail(err, "map launch");
            }
        }
        if (chosen == EIDM_ROUTE_GROUPED) {
            err = eidm::launch_grouped_split16(args, buf, device_cus(), stream);
            if (err != hipSuccess) return device_fail(err, "split-16 grouped launch");
        } else {
            err = eidm::launch_direct_split16(args, stream);
            if (err != hipSuccess) return device_fail(err, "split-16 direct launch");
        }
        return EIDM_OK;
    }
    if (chosen == EIDM_ROUTE_GROUPED) {
        if (build_map) {
            err = eidm::launch_map(args.ids, args.m * args.top_k, args.n_experts, buf, stream);
            if (err != hipSuccess) return device_fail(err, "map launch");
        }
        err = eidm::launch_grouped(args, buf, device_cus(), stream);
        if (err != hipSuccess) return device_fail(err, "grouped launch");
    } else {
        err = eidm::launch_direct(args, stream);
        if (err != hipSuccess) return device_fail(err, "direct launch");
    }
    return EIDM_OK;
}

int check_route_args(const float* logits, uint32_t m, uint32_t n_experts, uint32_t top_k,
                     const uint32_t* ids, const float* gates) {
    if (!logits || !ids) return api_fail(EIDM_E_INVALID, "logits or ids is NULL");
    if (!m || !n_experts || !top_k) return api_fail(EIDM_E_INVALID, "zero dimension");
    if (n_experts > eidm::kMaxExperts)
        return api_fail(EIDM_E_UNSUPPORTED, "n_experts %u above the supported %u", n_experts,
                    eidm::kMaxExperts);
    if (top_k > n_experts) return api_fail(EIDM_E_INVALID, "top_k %u above n_experts %u", top_k, n_experts);
    if (top_k > eidm::kMaxRouterTopK)
        return api_fail(EIDM_E_UNSUPPORTED, "router top_k %u above the supported %u", top_k,
                    eidm::kMaxRouterTopK);
    uint64_t tmp;
    if (!mul_ok(m, n_experts, &tmp) || tmp > (1ull << 40)) return api_fail(EIDM_E_INVALID, "m*n_experts too large");
    if ((uint64_t)m + 3 > kIndexLimit * 4) return api_fail(EIDM_E_UNSUPPORTED, "m too large");
    if (!aligned(logits, 4) || !aligned(ids, 4) || (gates && !aligned(gates, 4)))
        return api_fail(EIDM_E_ALIGN, "logits, ids and gates must be 4-byte aligned");
    return EIDM_OK;
}

int check_combine_args(uint32_t m, uint32_t top_k, uint32_t n, const float* y, const float* gates,
                       const float* out) {
    if (!y || !gates || !out) return api_fail(EIDM_E_INVALID, "y, gates or out is NULL");
    if (!m || !top_k || !n) return api_fail(EIDM_E_INVALID, "zero dimension");
    uint64_t t;
    if (!mul_ok(m, top_k, &t) || !mul_ok(t, n, &t)) return api_fail(EIDM_E_INVALID, "y size overflows");
    if (!aligned(y, 4) || !aligned(gates, 4) || !aligned(out, 4))
        return api_fail(EIDM_E_ALIGN, "y, gates and out must be 4-byte aligned");
    return EIDM_OK;
}

}  // namespace

extern "C" {

int eidm_abi_version(void) { return EIDM_ABI_VERSION; }

const char* eidm_last_error(void) { return g_error.c_str(); }

int eidm_last_dispatch(eidm_dispatch* out) {
    if (!out) return api_fail(EIDM_E_INVALID, "dispatch receipt is NULL");
    if (out->struct_size != sizeof(eidm_dispatch))
        return api_fail(EIDM_E_INVALID, "dispatch.struct_size is %u, expected %zu", out->struct_size,
                        sizeof(eidm_dispatch));
    *out = g_receipt;
    out->struct_size = sizeof(eidm_dispatch);
    return ok();
}

int eidm_query(const eidm_shape* shape, int route, eidm_requirements* out) {
    if (!out) return api_fail(EIDM_E_INVALID, "requirements is NULL");
    if (out->struct_size != sizeof(eidm_requirements))
        return api_fail(EIDM_E_INVALID, "requirements.struct_size is %u, expected %zu", out->struct_size,
                    sizeof(eidm_requirements));
    Plan p;
    int rc = check_shape(shape, &p);
    if (rc) return rc;
    int chosen = 0;
    rc = resolve_route(shape, p, route, false, 0, &chosen);
    if (rc) return rc;
    out->route = chosen;
    out->required_weight_bytes = p.required_weight_bytes;
    out->input_elements = p.input_elements;
    out->ids_elements = p.routed;
    out->output_elements = p.output_elements;
    out->scratch_bytes = chosen == EIDM_ROUTE_GROUPED ? p.grouped_scratch : p.direct_scratch;
    out->grouped_legal = 1;
    out->reserved0 = 0;
    return ok();
}

uint64_t eidm_map_scratch_bytes(uint32_t m, uint32_t top_k, uint32_t n_experts) {
    uint64_t routed;
    if (!mul_ok(m, top_k, &routed)) return 0;
    return eidm::map_hist_elements(routed, n_experts) * 4;
}

int eidm_route_topk(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                    uint32_t top_k, int renormalize, uint32_t* ids, float* gates, void* stream) {
    eidm::ReceiptScope receipt;
    int rc = check_route_args(logits, m, n_experts, top_k, ids, gates);
    if (rc) return rc;
    if (bias && !aligned(bias, 4)) return api_fail(EIDM_E_ALIGN, "bias must be 4-byte aligned");
    hipError_t err = eidm::launch_route(logits, bias, m, n_experts, top_k, renormalize, ids, gates,
                                        static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return device_fail(err, "route launch");
    return ok();
}

int eidm_map(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts, uint32_t* counts,
             uint32_t* offsets, uint32_t* rows, void* scratch, uint64_t scratch_bytes, void* stream) {
    eidm::ReceiptScope receipt;
    if (!ids || !counts || !offsets || !rows) return api_fail(EIDM_E_INVALID, "a map buffer is NULL");
    if (!m || !top_k || !n_experts) return api_fail(EIDM_E_INVALID, "zero dimension");
    if (n_experts > eidm::kMaxExperts)
        return api_fail(EIDM_E_UNSUPPORTED, "n_experts %u above the supported %u", n_experts,
                    eidm::kMaxExperts);
    uint64_t routed;
    if (!mul_ok(m, top_k, &routed) || routed > kIndexLimit)
        return api_fail(EIDM_E_UNSUPPORTED, "m*top_k at or above 2^31");
    const uint64_t need = eidm::map_hist_elements(routed, n_experts) * 4;
    if (!scratch || scratch_bytes < need)
        return api_fail(EIDM_E_SIZE, "map needs %llu bytes of scratch", (unsigned long long)need);
    if (!aligned(scratch, 4) || !aligned(ids, 4) || !aligned(counts, 4) || !aligned(offsets, 4) ||
        !aligned(rows, 4))
        return api_fail(EIDM_E_ALIGN, "map buffers must be 4-byte aligned");
    eidm::MapBuffers buf{static_cast<uint32_t*>(scratch), counts, offsets, rows};
    hipError_t err = eidm::launch_map(ids, (uint32_t)routed, n_experts, buf,
                                      static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return device_fail(err, "map launch");
    return ok();
}

int eidm_validate_ids(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts,
                      int multiplicity, int32_t* bad_index_out, void* stream) {
    eidm::ReceiptScope receipt;
    static std::mutex serial;  // the kernel reports through one device word
    if (!ids || !bad_index_out) return api_fail(EIDM_E_INVALID, "ids or bad_index_out is NULL");
    if (!m || !top_k || !n_experts) return api_fail(EIDM_E_INVALID, "zero dimension");
    if (multiplicity != EIDM_IDS_DISTINCT_PER_TOKEN && multiplicity != EIDM_IDS_MAY_REPEAT)
        return api_fail(EIDM_E_INVALID, "unknown id multiplicity %d", multiplicity);
    uint64_t routed;
    if (!mul_ok(m, top_k, &routed) || routed > kIndexLimit)
        return api_fail(EIDM_E_UNSUPPORTED, "m*top_k at or above 2^31");
    if (!aligned(ids, 4)) return api_fail(EIDM_E_ALIGN, "ids must be 4-byte aligned");
    int first_bad = -1;
    {
        std::lock_guard<std::mutex> lock(serial);
        const hipError_t err = eidm::run_validate(ids, m, top_k, n_experts,
                                                  multiplicity == EIDM_IDS_DISTINCT_PER_TOKEN,
                                                  static_cast<hipStream_t>(stream), &first_bad);
        if (err != hipSuccess) return device_fail(err, "id validation");
    }
    *bad_index_out = first_bad;
    if (first_bad >= 0)
        return api_fail(EIDM_E_IDS, "ids[%d] (token %u, slot %u) names no expert or repeats an earlier slot",
                    first_bad, (unsigned)(first_bad / top_k), (unsigned)(first_bad % top_k));
    return ok();
}

int eidm_matmul_id(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                   const float* input, const uint32_t* ids, float* output, void* scratch,
                   uint64_t scratch_bytes, void* stream, int* route_taken) {
    eidm::ReceiptScope receipt;
    eidm::MatmulArgs args{};
    eidm::MapBuffers buf{};
    int chosen = 0;
    int rc = prepare_matmul(shape, route, weights, weight_bytes, input, ids, output, scratch,
                            scratch_bytes, &args, &buf, &chosen);
    if (rc) return rc;
    rc = run_matmul(args, buf, chosen, static_cast<hipStream_t>(stream));
    if (rc) return rc;
    eidm::receipt_route(chosen);
    if (route_taken) *route_taken = chosen;
    return ok();
}

}  // extern "C"

namespace eidm {

// The map lives at offsets of the Grouped scratch that depend only on the
// routed-row count and the expert count, so calls over the same ids, routed
// rows and experts with the same scratch can share one map.
int matmul_id_shared_map(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                         const float* input, const uint32_t* ids, float* output, void* scratch,
                         uint64_t scratch_bytes, hipStream_t stream, bool* map_ready, int* route_taken) {
    MatmulArgs args{};
    MapBuffers buf{};
    int chosen = 0;
    int rc = prepare_matmul(shape, route, weights, weight_bytes, input, ids, output, scratch,
                            scratch_bytes, &args, &buf, &chosen);
    if (rc) return rc;
    const bool grouped = chosen == EIDM_ROUTE_GROUPED;
    rc = run_matmul(args, buf, chosen, stream, !(grouped && *map_ready));
    if (rc) return rc;
    receipt_route(chosen);
    if (grouped) *map_ready = true;
    if (route_taken) *route_taken = chosen;
    return ok();
}

}  // namespace eidm

extern "C" {

int eidm_combine(uint32_t m, uint32_t top_k, uint32_t n, const float* y, const float* gates,
                 float* out, void* stream) {
    eidm::ReceiptScope receipt;
    int rc = check_combine_args(m, top_k, n, y, gates, out);
    if (rc) return rc;
    hipError_t err = eidm::launch_combine(m, top_k, n, y, gates, out, static_cast<hipStream_t>(stream));
    if (err != hipSuccess) return device_fail(err, "combine launch");
    return ok();
}

int eidm_moe_forward(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                     const float* input, const float* logits, const float* bias, int renormalize,
                     uint32_t* ids, float* gates, float* y, float* out, void* scratch,
                     uint64_t scratch_bytes, void* stream, int* route_taken) {
    eidm::ReceiptScope receipt;
    eidm::MatmulArgs args{};
    eidm::MapBuffers buf{};
    int chosen = 0;
    // prepare_matmul checks shape (struct_size first) before any field is read
    int rc = prepare_matmul(shape, route, weights, weight_bytes, input, ids, y, scratch,
                            scratch_bytes, &args, &buf, &chosen);
    if (rc) return rc;
    if (shape->id_multiplicity != EIDM_IDS_DISTINCT_PER_TOKEN)
        return api_fail(EIDM_E_INVALID, "the router produces distinct ids; use DISTINCT_PER_TOKEN");
    if (!gates) return api_fail(EIDM_E_INVALID, "gates is NULL");
    rc = check_route_args(logits, shape->m, shape->n_experts, shape->top_k, ids, gates);
    if (rc) return rc;
    if (bias && !aligned(bias, 4)) return api_fail(EIDM_E_ALIGN, "bias must be 4-byte aligned");
    rc = check_combine_args(shape->m, shape->top_k, shape->n, y, gates, out);
    if (rc) return rc;
    hipStream_t st = static_cast<hipStream_t>(stream);
    if (chosen == EIDM_ROUTE_DIRECT && shape->arith == EIDM_ARITH_F32 &&
        eidm::moe_direct_supported(shape->top_k, shape->n_experts)) {
        // one kernel: route, Direct matmul and combine per (token, column group)
        const hipError_t err = eidm::launch_moe_direct(args, logits, bias, renormalize, ids, gates, out, device_cus(), st);
        if (err != hipSuccess) return device_fail(err, "fused route/Direct/combine launch");
        eidm::receipt_route(chosen);
        if (route_taken) *route_taken = chosen;
        return ok();
    }
    hipError_t err = eidm::launch_route(logits, bias, shape->m, shape->n_experts, shape->top_k,
                                        renormalize, ids, gates, st);
    if (err != hipSuccess) return device_fail(err, "route launch");
    rc = run_matmul(args, buf, chosen, st);
    if (rc) return rc;
    err = eidm::launch_combine(shape->m, shape->top_k, shape->n, y, gates, out, st);
    if (err != hipSuccess) return device_fail(err, "combine launch");
    eidm::receipt_route(chosen);
    if (route_taken) *route_taken = chosen;
    return ok();
}

}  // extern "C"
