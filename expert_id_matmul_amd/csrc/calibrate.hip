// calibrate.hip -- activation-time choice between the Direct and Grouped
// forms for exact shapes, and the frozen plan that serves that choice.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs:
//   * fn calibration_buffers: the calibration inputs -- adversarial
//     activations (eight bases including 1 + 2^-23, scaled by
//     1 + ((17 i) mod 11) / 4096), the balanced and skewed routing profiles,
//     outputs poisoned with a guard past the end;
//   * fn calibrate_one_inner: per profile, a Direct proof, a Grouped proof,
//     a bitwise comparison of the two, then five timing rounds that
//     alternate which form runs first;
//   * the winner rule: Grouped is chosen only if, on both profiles, its
//     median wall time is at most 0.95 x Direct's, its 75th-percentile wall
//     time is below Direct's 25th percentile, and its median GPU time is at
//     most 1.02 x Direct's; a failed Direct proof aborts, any Grouped
//     failure or difference in bits keeps Direct;
//   * fn resolve_dense_matmul_id_auto_route: an exact calibrated shape
//     takes its frozen route; a shape that differs from a calibrated one
//     only in m takes Direct; anything else fails before any work is
//     enqueued;
//   * DenseMatmulIdCalibrationLimits, struct Budget, the budget checks of
//     fn calibrate_one_inner and fn downgrade_grouped_after_deadline: an
//     activation has an elapsed-time, case and submission budget; Grouped
//     is never chosen on evidence that the budget could not pay for in full
//     or that finished after the deadline.
// Every proof and timing sample is a synchronous round trip; calibration is
// an activation-time step, not part of the hot path.
#include <hip/hip_runtime.h>

#include <algorithm>
#include <chrono>
#include <cstring>
#include <mutex>
#include <string>
#include <vector>

#include "eidm.h"
#include "eidm_internal.hpp"

struct eidm_plan {
    std::mutex mu;
    bool frozen = false;
    struct Entry {
        eidm_shape shape;
        int route;
    };
    std::vector<Entry> entries;
    // activation budget: limits, the clock's start, distinct shapes that
    // entered calibration, host waits spent (or reserved by a call in flight)
    eidm_calibration_limits limits{sizeof(eidm_calibration_limits), 256, 6145, 0, 15000};
    std::chrono::steady_clock::time_point started = std::chrono::steady_clock::now();
    std::vector<eidm_shape> cases;
    uint32_t submissions = 0;
    bool calibrated = false;  // an eidm_calibrate has begun: the limits are fixed

    double elapsed_ms() const {
        return std::chrono::duration<double, std::milli>(std::chrono::steady_clock::now() - started).count();
    }
    bool past_deadline() const { return elapsed_ms() >= (double)limits.max_elapsed_ms; }
};

namespace {

using eidm::api_fail;
using eidm::api_ok;

constexpr uint32_t kPoison = 0x7fc000c7u;  // a quiet-NaN pattern no computed value takes
constexpr uint32_t kGuard = 16;            // poisoned elements past each output
constexpr int kTimingRounds = 5;
constexpr int kCounters = 6;
// host waits of one complete gate: the inputs, then per profile the Direct
// proof, the Grouped proof, the proof check and the timing samples
constexpr uint32_t kGateSubmissions = 1 + 2 * (3 + 2 * kTimingRounds);

bool same_base(const eidm_shape& a, const eidm_shape& b) {
    return a.weight_dtype == b.weight_dtype && a.n == b.n && a.k == b.k && a.top_k == b.top_k &&
           a.n_experts == b.n_experts && a.expert_stride_bytes == b.expert_stride_bytes &&
           a.input_layout == b.input_layout && a.id_multiplicity == b.id_multiplicity && a.arith == b.arith;
}

bool same_shape(const eidm_shape& a, const eidm_shape& b) { return same_base(a, b) && a.m == b.m; }

uint64_t align256(uint64_t v) { return (v + 255) & ~uint64_t(255); }

// Workspace sections (256-byte aligned): activations | ids of the two
// profiles | Direct output + guard | Grouped output + guard | grouped
// scratch | proof counters.
struct Layout {
    uint64_t x, ids0, ids1, yd, yg, scratch, counters, total;
    uint64_t input_elements, routed, output_elements, scratch_bytes;
    bool grouped_legal;
};

int layout_for(const eidm_shape* shape, Layout* l) {
    eidm_requirements rd{}, rg{};
    rd.struct_size = sizeof(rd);
    rg.struct_size = sizeof(rg);
    int rc = eidm_query(shape, EIDM_ROUTE_DIRECT, &rd);
    if (rc) return rc;
    l->grouped_legal = eidm_query(shape, EIDM_ROUTE_GROUPED, &rg) == EIDM_OK && rg.grouped_legal;
    l->input_elements = rd.input_elements;
    l->routed = rd.ids_elements;
    l->output_elements = rd.output_elements;
    // one scratch for both forms (the split-16 Direct form needs one too)
    l->scratch_bytes = l->grouped_legal && rg.scratch_bytes > rd.scratch_bytes ? rg.scratch_bytes : rd.scratch_bytes;
    uint64_t off = 0;
    l->x = off;
    off = align256(off + l->input_elements * 4);
    l->ids0 = off;
    off = align256(off + l->routed * 4);
    l->ids1 = off;
    off = align256(off + l->routed * 4);
    l->yd = off;
    off = align256(off + (l->output_elements + kGuard) * 4);
    l->yg = off;
    off = align256(off + (l->output_elements + kGuard) * 4);
    l->scratch = off;
    off = align256(off + l->scratch_bytes);
    l->counters = off;
    l->total = off + kCounters * sizeof(unsigned long long);
    return api_ok();
}

// The calibration activations (fn calibration_buffers): element i of the
// input takes base[(5 i + i / k) mod 8] scaled by 1 + ((17 i) mod 11) / 4096.
std::vector<float> adversarial_activations(uint64_t elements, uint32_t k) {
    uint32_t b2 = 0x3f800001u, b3 = 0xbf800001u;
    float base[8] = {1.0009766f, -1.0009766f, 0.0f, 0.0f, 0.33333334f, -0.14285715f, 0.000012345679f,
                     -0.000009765625f};
    std::memcpy(&base[2], &b2, 4);
    std::memcpy(&base[3], &b3, 4);
    std::vector<float> x(elements);
    for (uint64_t i = 0; i < elements; ++i) {
        const float scale = 1.0f + (float)((i * 17) % 11) / 4096.0f;
        x[i] = base[(i * 5 + i / k) % 8] * scale;
    }
    return x;
}

// Routing profiles (fn calibration_buffers).  Ids distinct per token:
// balanced ids (t + s) mod E, so every expert gets the same number of rows,
// and skewed ids s, so all the rows land on the first top_k experts.  Ids
// that may repeat: t mod E in every slot, for both profiles.
std::vector<uint32_t> profile_ids(uint32_t m, uint32_t top_k, uint32_t n_experts, int may_repeat, int skewed) {
    std::vector<uint32_t> ids((uint64_t)m * top_k);
    for (uint32_t t = 0; t < m; ++t)
        for (uint32_t s = 0; s < top_k; ++s)
            ids[(uint64_t)t * top_k + s] = may_repeat ? t % n_experts
                                           : skewed   ? s
                                                      : (uint32_t)(((uint64_t)t + s) % n_experts);
    return ids;
}

// fn verified_bits, for both outputs at once.  counters: [0] Direct
// elements still poisoned, [1] Grouped elements still poisoned, [2]
// elements whose bits differ, [3] guard elements overwritten, [4] Direct
// elements not finite, [5] Grouped elements not finite
__global__ __launch_bounds__(256) void proof_kernel(const uint32_t* __restrict__ yd, const uint32_t* __restrict__ yg,
                                                    uint64_t count, int with_grouped,
                                                    unsigned long long* __restrict__ counters) {
    unsigned long long c[kCounters] = {0, 0, 0, 0, 0, 0};
    for (uint64_t i = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; i < count + kGuard;
         i += (uint64_t)gridDim.x * blockDim.x) {
        const uint32_t d = yd[i];
        const uint32_t g = with_grouped ? yg[i] : kPoison;
        if (i < count) {
            // exponent all ones: an infinity or a NaN (the poison is a NaN
            // too but is counted on its own)
            c[0] += d == kPoison;
            c[4] += d != kPoison && (d & 0x7f800000u) == 0x7f800000u;
            c[1] += with_grouped && g == kPoison;
            c[5] += with_grouped && g != kPoison && (g & 0x7f800000u) == 0x7f800000u;
            c[2] += with_grouped && d != g;
        } else {
            c[3] += d != kPoison || g != kPoison;
        }
    }
    for (int j = 0; j < kCounters; ++j)
        if (c[j]) atomicAdd(&counters[j], c[j]);
}

double pick(std::vector<double> v, int which) {  // 0: p25, 1: median, 2: p75 (the page's picks)
    std::sort(v.begin(), v.end());
    const size_t n = v.size();
    if (which == 0) return v[(n - 1) / 4];
    if (which == 1) return v[n / 2];
    return v[3 * (n - 1) / 4];
}

int hip_fail(hipError_t err, const char* what) {
    return api_fail(EIDM_E_DEVICE, "%s: %s", what, hipGetErrorString(err));
}

}  // namespace

extern "C" {

eidm_plan* eidm_plan_create(void) { return new (std::nothrow) eidm_plan(); }

void eidm_plan_destroy(eidm_plan* plan) { delete plan; }

int eidm_plan_set_limits(eidm_plan* plan, const eidm_calibration_limits* limits) {
    if (!plan || !limits) return api_fail(EIDM_E_INVALID, "plan or limits is NULL");
    if (limits->struct_size != sizeof(eidm_calibration_limits))
        return api_fail(EIDM_E_INVALID, "limits struct_size %u, expected %zu", limits->struct_size,
                        sizeof(eidm_calibration_limits));
    if (limits->max_elapsed_ms == 0 || limits->max_cases == 0 || limits->max_submissions == 0)
        return api_fail(EIDM_E_INVALID, "calibration limits must be nonzero");
    std::lock_guard<std::mutex> lock(plan->mu);
    if (plan->frozen || plan->calibrated)
        return api_fail(EIDM_E_INVALID, "limits are fixed once calibration has begun");
    plan->limits = *limits;
    plan->started = std::chrono::steady_clock::now();
    return api_ok();
}

int eidm_plan_freeze(eidm_plan* plan, uint32_t* downgraded) {
    if (!plan) return api_fail(EIDM_E_INVALID, "plan is NULL");
    std::lock_guard<std::mutex> lock(plan->mu);
    uint32_t changed = 0;
    if (!plan->frozen && plan->elapsed_ms() > (double)plan->limits.max_elapsed_ms) {
        // fn downgrade_grouped_after_deadline: a plan published after the
        // deadline holds no Grouped route
        for (auto& e : plan->entries)
            if (e.route == EIDM_ROUTE_GROUPED) {
                e.route = EIDM_ROUTE_DIRECT;
                ++changed;
            }
    }
    plan->frozen = true;
    if (downgraded) *downgraded = changed;
    return api_ok();
}

int eidm_plan_route(const eidm_plan* plan, const eidm_shape* shape, int* route) {
    if (!plan || !shape || !route) return api_fail(EIDM_E_INVALID, "plan, shape or route is NULL");
    eidm_plan* p = const_cast<eidm_plan*>(plan);
    std::lock_guard<std::mutex> lock(p->mu);
    bool base = false;
    for (const auto& e : p->entries) {
        if (same_shape(e.shape, *shape)) {
            *route = e.route;
            return api_ok();
        }
        base = base || same_base(e.shape, *shape);
    }
    if (base) {  // an admitted base with an unseen m
        *route = EIDM_ROUTE_DIRECT;
        return api_ok();
    }
    return api_fail(EIDM_E_UNSUPPORTED, "shape (m=%u n=%u k=%u top_k=%u n_experts=%u) was not calibrated",
                    shape->m, shape->n, shape->k, shape->top_k, shape->n_experts);
}

uint64_t eidm_calibration_workspace_bytes(const eidm_shape* shape) {
    Layout l{};
    if (!shape || layout_for(shape, &l) != EIDM_OK) return 0;
    return l.total;
}

int eidm_calibrate(eidm_plan* plan, const eidm_shape* shape, const void* weights, uint64_t weight_bytes,
                   void* workspace, uint64_t workspace_bytes, void* stream, eidm_calibration* receipt) {
    eidm::ReceiptScope dispatch_receipt;
    if (!plan || !shape || !weights || !workspace || !receipt)
        return api_fail(EIDM_E_INVALID, "plan, shape, weights, workspace or receipt is NULL");
    if (receipt->struct_size != sizeof(eidm_calibration))
        return api_fail(EIDM_E_INVALID, "receipt struct_size %u, expected %zu", receipt->struct_size,
                        sizeof(eidm_calibration));
    Layout l{};
    int rc = layout_for(shape, &l);
    if (rc) return rc;
    if (workspace_bytes < l.total)
        return api_fail(EIDM_E_SIZE, "calibration needs %llu bytes of workspace, got %llu",
                        (unsigned long long)l.total, (unsigned long long)workspace_bytes);
    if (reinterpret_cast<uintptr_t>(workspace) % 256)
        return api_fail(EIDM_E_ALIGN, "the workspace must be 256-byte aligned");

    eidm_calibration out{};
    out.struct_size = sizeof(out);
    out.grouped_legal = l.grouped_legal;
    out.route = EIDM_ROUTE_DIRECT;

    // The decision is stored and the receipt filled by `finish`; `reserved`
    // host waits were taken from the plan's budget at the start and are
    // given back, less what the call used.
    uint32_t reserved = 0;
    auto finish = [&](int reason) -> int {
        out.reason = reason;
        out.route = reason == EIDM_CAL_GROUPED_WINS ? EIDM_ROUTE_GROUPED : EIDM_ROUTE_DIRECT;
        std::lock_guard<std::mutex> lock(plan->mu);
        plan->submissions = plan->submissions - reserved + out.submissions;
        reserved = 0;
        if (plan->frozen) return api_fail(EIDM_E_INVALID, "the plan was frozen during calibration");
        bool replaced = false;
        for (auto& e : plan->entries)
            if (same_shape(e.shape, *shape)) {
                e.route = out.route;
                replaced = true;
            }
        if (!replaced) plan->entries.push_back({*shape, out.route});
        *receipt = out;
        return api_ok();
    };
    // a failed call gives back its reservation and keeps what it spent
    struct Refund {
        eidm_plan* plan;
        uint32_t* reserved;
        const uint32_t* used;
        ~Refund() {
            if (!*reserved) return;
            std::lock_guard<std::mutex> lock(plan->mu);
            plan->submissions = plan->submissions - *reserved + *used;
        }
    } refund{plan, &reserved, &out.submissions};

    {  // admission: frozen plan, case limit, then the budget for a complete gate
        std::lock_guard<std::mutex> lock(plan->mu);
        if (plan->frozen) return api_fail(EIDM_E_INVALID, "the plan is frozen");
        bool known = false;
        for (const auto& c : plan->cases) known = known || same_shape(c, *shape);
        if (!known && plan->cases.size() >= plan->limits.max_cases)
            return api_fail(EIDM_E_INVALID, "calibration of a new shape beyond the plan's %u cases",
                            plan->limits.max_cases);
        if (!known) plan->cases.push_back(*shape);
        plan->calibrated = true;
        if (l.grouped_legal && plan->submissions + kGateSubmissions <= plan->limits.max_submissions &&
            !plan->past_deadline()) {
            reserved = kGateSubmissions;
            plan->submissions += reserved;
        }
    }
    if (!l.grouped_legal) return finish(EIDM_CAL_GROUPED_NOT_LEGAL);  // Direct only: no GPU work
    if (!reserved) return finish(EIDM_CAL_BUDGET);                    // no complete gate fits

    hipStream_t st = static_cast<hipStream_t>(stream);
    uint8_t* ws = static_cast<uint8_t*>(workspace);
    float* x = reinterpret_cast<float*>(ws + l.x);
    uint32_t* ids[2] = {reinterpret_cast<uint32_t*>(ws + l.ids0), reinterpret_cast<uint32_t*>(ws + l.ids1)};
    float* yd = reinterpret_cast<float*>(ws + l.yd);
    float* yg = reinterpret_cast<float*>(ws + l.yg);
    void* scratch = ws + l.scratch;  // l.scratch_bytes of it
    unsigned long long* counters = reinterpret_cast<unsigned long long*>(ws + l.counters);
    const int may_repeat = shape->id_multiplicity == EIDM_IDS_MAY_REPEAT;

    {  // inputs: one host wait
        const std::vector<float> hx = adversarial_activations(l.input_elements, shape->k);
        const std::vector<uint32_t> h0 = profile_ids(shape->m, shape->top_k, shape->n_experts, may_repeat, 0);
        const std::vector<uint32_t> h1 = profile_ids(shape->m, shape->top_k, shape->n_experts, may_repeat, 1);
        hipError_t err = hipMemcpyAsync(x, hx.data(), hx.size() * 4, hipMemcpyHostToDevice, st);
        if (err == hipSuccess) err = hipMemcpyAsync(ids[0], h0.data(), h0.size() * 4, hipMemcpyHostToDevice, st);
        if (err == hipSuccess) err = hipMemcpyAsync(ids[1], h1.data(), h1.size() * 4, hipMemcpyHostToDevice, st);
        if (err == hipSuccess) err = hipStreamSynchronize(st);
        ++out.submissions;
        if (err != hipSuccess) return hip_fail(err, "calibration inputs");
    }

    hipEvent_t ev[2];
    if (hipEventCreate(&ev[0]) != hipSuccess) return api_fail(EIDM_E_DEVICE, "event create");
    if (hipEventCreate(&ev[1]) != hipSuccess) {
        (void)hipEventDestroy(ev[0]);
        return api_fail(EIDM_E_DEVICE, "event create");
    }
    struct Events {
        hipEvent_t* e;
        ~Events() {
            (void)hipEventDestroy(e[0]);
            (void)hipEventDestroy(e[1]);
        }
    } guard_events{ev};

    bool grouped_ok = true;
    bool identical = true;
    int reason = EIDM_CAL_GROUPED_WINS;
    const uint64_t out_words = l.output_elements + kGuard;

    // one call of one form on profile p, one host wait; wall and GPU
    // microseconds
    auto call = [&](int route, int p, double* wall_us, double* gpu_us) -> int {
        float* y = route == EIDM_ROUTE_DIRECT ? yd : yg;
        const auto t0 = std::chrono::steady_clock::now();
        hipError_t err = hipEventRecord(ev[0], st);
        if (err != hipSuccess) return hip_fail(err, "event record");
        int r = eidm_matmul_id(shape, route, weights, weight_bytes, x, ids[p], y, l.scratch_bytes ? scratch : nullptr,
                               l.scratch_bytes, stream, nullptr);
        if (r) return r;
        err = hipEventRecord(ev[1], st);
        if (err == hipSuccess) err = hipStreamSynchronize(st);
        ++out.submissions;
        if (err != hipSuccess) return hip_fail(err, "calibration call");
        const auto t1 = std::chrono::steady_clock::now();
        float ms = 0.0f;
        err = hipEventElapsedTime(&ms, ev[0], ev[1]);
        if (err != hipSuccess) return hip_fail(err, "event time");
        if (wall_us) *wall_us = std::chrono::duration<double, std::micro>(t1 - t0).count();
        if (gpu_us) *gpu_us = ms * 1e3;
        return EIDM_OK;
    };
    // the Direct form's failures end the calibration, keeping the inner error
    auto direct_failed = [&](int code, const char* what, int p) -> int {
        const std::string inner = eidm_last_error();
        return api_fail(code, "%s failed (profile %d): %s", what, p, inner.c_str());
    };

    for (int p = 0; p < 2 && grouped_ok; ++p) {
        // proofs: poisoned outputs, one call of each form, then the device check
        hipError_t err = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(yd), (int)kPoison, out_words, st);
        if (err == hipSuccess)
            err = hipMemsetD32Async(reinterpret_cast<hipDeviceptr_t>(yg), (int)kPoison, out_words, st);
        if (err == hipSuccess) err = hipMemsetAsync(counters, 0, kCounters * sizeof(unsigned long long), st);
        if (err != hipSuccess) return hip_fail(err, "poison");
        rc = call(EIDM_ROUTE_DIRECT, p, nullptr, nullptr);
        if (rc) return direct_failed(rc, "Direct proof", p);
        if (call(EIDM_ROUTE_GROUPED, p, nullptr, nullptr) != EIDM_OK) {
            grouped_ok = identical = false;
            reason = EIDM_CAL_GROUPED_FAILED;
        }
        const uint64_t blocks = std::min<uint64_t>((out_words + 255) / 256, 4096);
        hipLaunchKernelGGL(proof_kernel, dim3((uint32_t)blocks), dim3(256), 0, st,
                           reinterpret_cast<const uint32_t*>(yd), reinterpret_cast<const uint32_t*>(yg),
                           l.output_elements, grouped_ok ? 1 : 0, counters);
        unsigned long long c[kCounters] = {0, 0, 0, 0, 0, 0};
        err = eidm::launched(EIDM_KERNEL_PROOF, (uint32_t)blocks, 256, 0);
        if (err == hipSuccess) err = hipMemcpyAsync(c, counters, sizeof(c), hipMemcpyDeviceToHost, st);
        if (err == hipSuccess) err = hipStreamSynchronize(st);
        ++out.submissions;
        if (err != hipSuccess) return hip_fail(err, "proof check");
        if (c[0] != 0 || c[3] != 0 || c[4] != 0)
            return api_fail(EIDM_E_DEVICE,
                            "Direct proof failed (profile %d): %llu outputs unwritten, %llu not finite, %llu guard "
                            "elements overwritten",
                            p, c[0], c[4], c[3]);
        if (grouped_ok && (c[1] != 0 || c[5] != 0)) {
            grouped_ok = identical = false;
            reason = EIDM_CAL_GROUPED_FAILED;
        } else if (grouped_ok && c[2] != 0) {
            grouped_ok = identical = false;
            reason = EIDM_CAL_NOT_IDENTICAL;
        }
        if (!grouped_ok) break;

        // timing: five rounds, the first form alternating; the deadline is
        // checked before every sample
        std::vector<double> dw, dg, gw, gg;
        for (int round = 0; round < kTimingRounds && grouped_ok; ++round) {
            const int first = round % 2 == 0 ? EIDM_ROUTE_DIRECT : EIDM_ROUTE_GROUPED;
            for (int j = 0; j < 2 && grouped_ok; ++j) {
                const int route = j == 0 ? first : (first == EIDM_ROUTE_DIRECT ? EIDM_ROUTE_GROUPED : EIDM_ROUTE_DIRECT);
                if (plan->past_deadline()) return finish(EIDM_CAL_BUDGET);
                double w = 0.0, g = 0.0;
                rc = call(route, p, &w, &g);
                if (rc) {
                    if (route == EIDM_ROUTE_DIRECT) return direct_failed(rc, "Direct timing", p);
                    grouped_ok = false;
                    reason = EIDM_CAL_GROUPED_FAILED;
                    break;
                }
                (route == EIDM_ROUTE_DIRECT ? dw : gw).push_back(w);
                (route == EIDM_ROUTE_DIRECT ? dg : gg).push_back(g);
            }
        }
        if (!grouped_ok) break;
        out.direct_wall_p25[p] = pick(dw, 0);
        out.direct_wall_median[p] = pick(dw, 1);
        out.direct_wall_p75[p] = pick(dw, 2);
        out.direct_gpu_median[p] = pick(dg, 1);
        out.grouped_wall_p25[p] = pick(gw, 0);
        out.grouped_wall_median[p] = pick(gw, 1);
        out.grouped_wall_p75[p] = pick(gw, 2);
        out.grouped_gpu_median[p] = pick(gg, 1);
        // the winner rule, checked profile by profile (the first failed test is the reason)
        if (reason == EIDM_CAL_GROUPED_WINS) {
            if (!(out.grouped_wall_median[p] <= 0.95 * out.direct_wall_median[p])) reason = EIDM_CAL_WALL_MEDIAN;
            else if (!(out.grouped_wall_p75[p] < out.direct_wall_p25[p])) reason = EIDM_CAL_WALL_QUARTILES;
            else if (!(out.grouped_gpu_median[p] <= 1.02 * out.direct_gpu_median[p])) reason = EIDM_CAL_GPU_MEDIAN;
        }
    }

    out.bit_identical = identical ? 1 : 0;
    // the last timed sample may end after the deadline: no Grouped choice
    // from evidence completed without authority
    if (reason == EIDM_CAL_GROUPED_WINS && plan->past_deadline()) reason = EIDM_CAL_BUDGET;
    return finish(reason);
}

int eidm_matmul_id_planned(const eidm_plan* plan, const eidm_shape* shape, const void* weights,
                           uint64_t weight_bytes, const float* input, const uint32_t* ids, float* output,
                           void* scratch, uint64_t scratch_bytes, void* stream, int* route_taken) {
    eidm::ReceiptScope dispatch_receipt;
    int route = 0;
    const int rc = eidm_plan_route(plan, shape, &route);
    if (rc) return rc;
    return eidm_matmul_id(shape, route, weights, weight_bytes, input, ids, output, scratch, scratch_bytes,
                          stream, route_taken);
}

}  // extern "C"
