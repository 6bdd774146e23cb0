/*
 * eidm.h -- C ABI of libeidm.so: the mixture-of-experts expert-ID matmul
 * (matmul_id) path on one AMD Instinct MI355X (gfx950).
 *
 * The path, for m tokens each routed to top_k of n_experts experts:
 *   1. route    sigmoid + selection-bias top-k router -> ids, gates
 *   2. map      per-expert lists of routed rows (grouped form only)
 *   3. matmul   y[r, :] = W[ids[r]] . x_row(r) for every routed row
 *               r = t*top_k + s, in one of two forms that give identical
 *               bits: Direct (one routed row at a time, weight streaming)
 *               and Grouped (each expert's gathered rows as one tile job)
 *   4. combine  out[t, :] = sum_s gate[t, s] * y[t*top_k + s, :]
 *
 * Sources (docs.rs source views):
 *   mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs -- the shape key
 *     (struct DenseMatmulIdShape), the two routes and their required
 *     bit identity (the value-independence theorem statement), the weight
 *     extent and alignment checks (fn validate_cases), the input layouts,
 *     id multiplicity and routing profiles (fn calibration_buffers), the
 *     map pass and grouped scratch sized by (n_experts, m)
 *     (fn expected_dispatches, DenseMatmulIdScratch::new).
 *   cortiq-engine 0.7.7, src/mimo_moe.rs -- sigmoid + selection-bias
 *     routing with renormalised gates p[e]/wsum (module doc, Dynamic::run,
 *     the bank_tests model arch).
 *   hf2q, src/inference/models/qwen35/dense_ffn_arena.rs -- routed-row
 *     major ids/weights/y buffers and the weighted reduce (MoeFfnArena).
 *
 * Conventions (all entry points):
 *   - Every pointer marked "device" is caller-owned device memory (for
 *     example from hipMalloc or a torch CUDA tensor's data_ptr()).  The
 *     library never allocates, frees or retains caller memory; buffers must
 *     stay alive until the stream has passed the enqueued work.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Work is enqueued asynchronously on it; nothing synchronises.
 *   - All arguments are validated on the host before anything is enqueued.
 *     On a validation error the call returns a negative eidm_status,
 *     enqueues nothing, and eidm_last_error() describes the failure.  A
 *     call of several steps (eidm_moe_forward, eidm_moe_ffn, a Grouped
 *     eidm_matmul_id) that gets EIDM_E_DEVICE from a later launch has
 *     already enqueued its earlier steps; its outputs (ids, gates, y,
 *     out) are then undefined, and eidm_last_dispatch() lists what was
 *     enqueued.
 *   - Sizes use overflow-checked products (an overflow is EIDM_E_INVALID).
 *   - Entry points are reentrant; a scratch buffer belongs to one call in
 *     flight at a time.
 *   - Floating point: activations, gates and outputs are f32; weights are
 *     native f32/f16/bf16, widened exactly to f32; every product is
 *     accumulated with f32 fused multiply-add.
 */
#ifndef EIDM_H
#define EIDM_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define EIDM_ABI_VERSION 2

/* Native weight scalar type (DenseMatmulIdShape.weight_dtype). */
typedef enum eidm_dtype {
    EIDM_DTYPE_F32 = 0,
    EIDM_DTYPE_F16 = 1,
    EIDM_DTYPE_BF16 = 2
} eidm_dtype;

/* Input rows: one per token shared by its top_k slots ([m, k]), or one per
 * routed row ([m*top_k, k]) (DenseMatmulIdInputLayout). */
typedef enum eidm_layout {
    EIDM_LAYOUT_SHARED_PER_TOKEN = 0,
    EIDM_LAYOUT_SLOTTED = 1
} eidm_layout;

/* Whether one token's top_k ids are distinct (DenseMatmulIdMultiplicity). */
typedef enum eidm_multiplicity {
    EIDM_IDS_DISTINCT_PER_TOKEN = 0,
    EIDM_IDS_MAY_REPEAT = 1
} eidm_multiplicity;

/* The arithmetic of the matmul.  F32: native weights widened to f32, f32
 * fma in the fixed 16-slice order (see eidm_matmul_id).  SPLIT16: 16-bit
 * weights kept exact in their own type, each f32 activation split exactly
 * into three parts of that type, products on the 16-bit matrix core (the
 * value-independence theorem statement of dense_matmul_id_auto.rs: both
 * routes, one order).  Both routes give identical bits within a mode; the
 * modes differ from each other by rounding only. */
typedef enum eidm_arith {
    EIDM_ARITH_F32 = 0,
    EIDM_ARITH_SPLIT16 = 1
} eidm_arith;

/* Which form of the matmul runs (DenseMatmulIdRoute, plus AUTO). */
typedef enum eidm_route {
    EIDM_ROUTE_AUTO = 0,
    EIDM_ROUTE_DIRECT = 1,
    EIDM_ROUTE_GROUPED = 2
} eidm_route;

typedef enum eidm_status {
    EIDM_OK = 0,
    EIDM_E_INVALID = -1,     /* zero dimension, bad enum, null pointer, overflow */
    EIDM_E_UNSUPPORTED = -2, /* route not legal for the shape                    */
    EIDM_E_SIZE = -3,        /* weight extent or scratch too small              */
    EIDM_E_ALIGN = -4,       /* pointer or stride misaligned for its type        */
    EIDM_E_DEVICE = -5,      /* a HIP call failed                                */
    EIDM_E_IDS = -6          /* eidm_validate_ids found a bad id                 */
} eidm_status;

/*
 * The full shape key of one matmul_id case (DenseMatmulIdShape: weight
 * dtype, m, n, k, top_k, n_experts, expert stride, input layout, id
 * multiplicity).  Expert e's weight matrix is [n, k], row-major (k
 * contiguous), starting at byte e * expert_stride_bytes of the weight
 * buffer; the stride may include padding.  `arith` picks the arithmetic
 * (eidm_arith; 0 is the f32 order).  struct_size must be sizeof(eidm_shape).
 */
typedef struct eidm_shape {
    uint32_t struct_size;
    int32_t weight_dtype;        /* eidm_dtype */
    uint32_t m;                  /* tokens                     */
    uint32_t n;                  /* output columns per row     */
    uint32_t k;                  /* reduction length           */
    uint32_t top_k;              /* routed rows per token      */
    uint32_t n_experts;
    int32_t arith;               /* eidm_arith (0: F32)        */
    uint64_t expert_stride_bytes;
    int32_t input_layout;        /* eidm_layout                */
    int32_t id_multiplicity;     /* eidm_multiplicity          */
} eidm_shape;

/* What one case needs from the caller (host-only query). */
typedef struct eidm_requirements {
    uint32_t struct_size;        /* set by the caller: sizeof(eidm_requirements) */
    int32_t route;               /* the route the query resolved to             */
    uint64_t required_weight_bytes; /* (n_experts-1)*stride + n*k*sizeof(dtype)  */
    uint64_t input_elements;     /* f32: m*k (shared) or m*top_k*k (slotted)    */
    uint64_t ids_elements;       /* u32: m*top_k                                */
    uint64_t output_elements;    /* f32: m*top_k*n                              */
    uint64_t scratch_bytes;      /* device scratch the route needs (0: none)    */
    int32_t grouped_legal;       /* 1 when the Grouped route accepts the shape  */
    int32_t reserved0;
} eidm_requirements;

/* Kernels a call can launch (eidm_launch.kernel). */
typedef enum eidm_kernel {
    EIDM_KERNEL_ROUTE = 1,          /* sigmoid + bias top-k router                  */
    EIDM_KERNEL_MAP_ONE_PASS = 2,   /* id -> row map, one launch (small maps)        */
    EIDM_KERNEL_MAP_HISTOGRAM = 3,  /* id -> row map, first of two launches          */
    EIDM_KERNEL_MAP_SCATTER = 4,    /* id -> row map, second of two launches         */
    EIDM_KERNEL_DIRECT = 5,         /* Direct matmul_id                              */
    EIDM_KERNEL_GROUPED_16X16 = 6,  /* Grouped matmul_id, 16x16x1 matrix-core form   */
    EIDM_KERNEL_GROUPED_STREAM = 7, /* Grouped matmul_id, 4x4x1 streamed form        */
    EIDM_KERNEL_GROUPED_JOB = 8,    /* Grouped matmul_id, 4x4x1 per-job form         */
    EIDM_KERNEL_COMBINE = 9,        /* gate-weighted slot sum                        */
    EIDM_KERNEL_FUSED_DECODE = 10,  /* route + Direct + combine in one launch        */
    EIDM_KERNEL_SILU_MUL = 11,      /* expert FFN: silu(gate) * up                   */
    EIDM_KERNEL_VALIDATE = 12,      /* id table check                                */
    EIDM_KERNEL_PROOF = 13,         /* calibration proof check                       */
    EIDM_KERNEL_SPLIT_X = 14,       /* split-16: activations into three parts        */
    EIDM_KERNEL_DIRECT_SPLIT16 = 15,  /* split-16 Direct                             */
    EIDM_KERNEL_GROUPED_SPLIT16 = 16, /* split-16 Grouped                            */
    EIDM_KERNEL_MAP_SPLIT_X = 17      /* split-16 Grouped: the one-launch map and the
                                         activation split in one launch              */
} eidm_kernel;

/* One kernel launch: which kernel and its launch geometry (1-D grid of
 * `grid` blocks of `block` threads, `lds_bytes` of dynamic LDS). */
typedef struct eidm_launch {
    int32_t kernel;                 /* eidm_kernel */
    uint32_t grid;
    uint32_t block;
    uint32_t lds_bytes;
} eidm_launch;

#define EIDM_MAX_RECORDED_LAUNCHES 16

/* What the calling thread's last call enqueued (mlx-native
 * dense_matmul_id_auto.rs: the primitive's receipt {route, dispatch count}
 * and fn expected_dispatches, the launch geometry checked after each
 * encode). */
typedef struct eidm_dispatch {
    uint32_t struct_size;           /* set by the caller: sizeof(eidm_dispatch)         */
    int32_t route;                  /* eidm_route the call ran (0: none, or it failed)   */
    uint32_t dispatch_count;        /* kernel launches the call enqueued                 */
    uint32_t recorded;              /* entries of launches[] filled, in launch order     */
    eidm_launch launches[EIDM_MAX_RECORDED_LAUNCHES];
} eidm_dispatch;

/*
 * Host-only: the dispatch receipt of the last library call on the calling
 * thread (every entry point that can enqueue work starts a new one; calls a
 * library entry point makes internally add to the caller's).  A successful
 * eidm_matmul_id is 1 launch for Direct; for Grouped the map (1 or 2
 * launches) and the Grouped kernel, or the Grouped kernel alone when the
 * map is reused (the later projections of eidm_moe_ffn).  In the split-16
 * arithmetic the activation split comes first (Direct: 2 launches); for
 * Grouped it shares one launch with the map when the map takes its
 * one-launch form (then 2 launches, else split, map, Grouped).  An
 * eidm_moe_forward that runs Direct with top_k <= 16 is 1 fused launch.
 * Enqueues nothing.
 */
int eidm_last_dispatch(eidm_dispatch* out);

/* ABI version of the loaded library (EIDM_ABI_VERSION it was built with). */
int eidm_abi_version(void);

/* Description of the last error on the calling thread ("" if none). */
const char* eidm_last_error(void);

/*
 * Host-only: validate `shape` and report its buffer sizes and the scratch
 * the route needs.  `route` may be AUTO (the answer names the route AUTO
 * picks when given that scratch).  Dimensions must be non-zero, the stride
 * must cover one expert (n*k*size bytes) and be a multiple of the dtype
 * size, top_k <= n_experts for distinct ids.  Grouped is legal for both
 * multiplicities.  Enqueues nothing.
 */
int eidm_query(const eidm_shape* shape, int route, eidm_requirements* out);

/*
 * Router (cortiq-engine mimo_moe.rs: module doc, Dynamic::run and the
 * bank_tests arch with router_sigmoid and norm_topk_prob):
 *   s[t,e]   = sigmoid(logits[t,e]), rounded to f32
 *   sel[t,e] = s[t,e] + bias[e]  (one f32 add; bias may be NULL = 0)
 *   ids[t,j] = j-th largest sel of token t (j = 0..top_k-1); equal sel
 *              keeps the lower expert index first; ids are distinct
 *   gates[t,j] = s[t,ids[t,j]] / sum_j' s[t,ids[t,j']] (f32, sum in slot
 *              order) when renormalize != 0, else s[t,ids[t,j]]
 * logits: device f32 [m, n_experts]; bias: device f32 [n_experts] or NULL;
 * ids: device u32 [m, top_k]; gates: device f32 [m, top_k] (may be NULL).
 * Requires 1 <= top_k <= min(n_experts, 64) and n_experts <= 2048 (larger
 * values return EIDM_E_UNSUPPORTED).  Logits must be finite (a NaN
 * logit ranks below every finite one; the ids stay distinct and in range).
 */
int eidm_route_topk(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                    uint32_t top_k, int renormalize, uint32_t* ids, float* gates, void* stream);

/*
 * Id -> row map (the map pass of the grouped route, mlx-native
 * dense_matmul_id_auto.rs fn expected_dispatches): a stable counting sort
 * of the routed rows r = 0..m*top_k-1 by key min(ids[r], n_experts).
 *   counts  device u32 [n_experts+1]: rows per key (key n_experts = ids that
 *           name no expert)
 *   offsets device u32 [n_experts+2]: exclusive prefix sums of counts
 *   rows    device u32 [m*top_k]: the rows, grouped by key, ascending
 *           within each key
 *   scratch device, >= eidm_map_scratch_bytes(m, top_k, n_experts) bytes,
 *           4-byte aligned (per-block histograms; small maps, up to 16384
 *           routed rows, are built in one pass without it, but the size is
 *           required either way)
 * Results are exact and deterministic, the same for either form.  Requires
 * m*top_k < 2^31 and n_experts <= 2048.
 */
int eidm_map(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts,
             uint32_t* counts, uint32_t* offsets, uint32_t* rows, void* scratch,
             uint64_t scratch_bytes, void* stream);

/* Host-only: scratch bytes eidm_map needs (0 if m*top_k overflows). */
uint64_t eidm_map_scratch_bytes(uint32_t m, uint32_t top_k, uint32_t n_experts);

/*
 * The expert-ID matmul (mlx-native dense_matmul_id_auto.rs: the shape key,
 * the routes, the value-independence theorem statement):
 *   y[r, j] = sum_c widen(W_e[j, c]) * x_row(r)[c],  e = ids[r],
 *   r = t*top_k + s,  x_row(r) = input[t] (shared) or input[r] (slotted).
 * weights      device, >= required_weight_bytes, aligned to the dtype size
 * weight_bytes the extent the caller vouches for (checked against the shape)
 * input        device f32 [input_elements]
 * ids          device u32 [m, top_k]
 * output       device f32 [m*top_k, n]; every element is overwritten and
 *              nothing past it is written
 * scratch      device, >= scratch_bytes from eidm_query for the route (may
 *              be NULL for Direct); 256-byte aligned
 * route_taken  (optional host int*) receives the route that ran
 * Both routes give bit-identical outputs for the same inputs.  With
 * EIDM_ARITH_F32 the reduction over k is the same fixed order in both: k is
 * cut into granules of 8; granule g belongs to slice g mod 16; each slice
 * accumulates its products in ascending k with f32 fma from +0; the 16
 * slice sums are added pairwise as (s, s+8), then (s, s+4), (s, s+2),
 * (s, s+1).
 * With EIDM_ARITH_SPLIT16 (16-bit weights; k a multiple of 8; weights,
 * stride and input 16-byte aligned) each activation x is split into
 * p1 = rn(x), p2 = rn(x - p1), p3 = rn(x - p1 - p2) in the weight type
 * (exact for bf16; for f16, |x| must stay below 65504 and parts below
 * 2^-24 round), and k is cut into steps of 32 (zero past k, the step count
 * rounded up to a multiple of 4).  Per output, with v_mfma_f32_16x16x32 of
 * the weight type (its result does not depend on the tile position): a hi
 * chain from +0 over the p1 products of every step, a lo chain from +0 over
 * the p2 then p3 products of every step, y = hi + lo (one f32 add).
 * Measured on MI355X: per-output error below 3e-6 relative for k <= 4096
 * with N(0,1) activations.  Each expert's matrix and the split activations
 * must span less than 2 GiB.  Both routes then need scratch (eidm_query)
 * for the split activations.
 * An id >= n_experts makes its output row quiet NaN (no weights are read).
 * AUTO runs Grouped when it is legal, scratch covers it and the routed rows
 * average at least 2 per expert (m*top_k >= 2*n_experts); Direct otherwise.
 */
int eidm_matmul_id(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                   const float* input, const uint32_t* ids, float* output, void* scratch,
                   uint64_t scratch_bytes, void* stream, int* route_taken);

/*
 * eidm_matmul_id for callers that cannot allocate device memory (code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation):
 * the same computation and bits, with no scratch argument.  The scratch a
 * route needs (the Grouped route's id -> row map; with EIDM_ARITH_SPLIT16
 * the split activations of either route) lives in a device array the
 * library owns, 8 MiB per GPU, held from the first call on that GPU until
 * the process ends; the call itself allocates nothing.  Arguments as in
 * eidm_matmul_id (weights, input, ids and output are still the caller's).
 * DIRECT or GROUPED fails with EIDM_E_SIZE, before anything is enqueued,
 * when its scratch (eidm_query's scratch_bytes) exceeds 8 MiB; AUTO then
 * runs Direct.  Every call on one
 * GPU uses the same array, so calls whose work overlaps in time on one GPU
 * (several streams or host threads) race; issue them on one stream.
 */
int eidm_matmul_id_noalloc(const eidm_shape* shape, int route, const void* weights, uint64_t weight_bytes,
                           const float* input, const uint32_t* ids, float* output, void* stream,
                           int* route_taken);

/*
 * Gate-weighted sum over slots (cortiq-engine mimo_moe.rs Dynamic::run;
 * hf2q dense_ffn_arena.rs MoeFfnArena's weighted reduce):
 *   out[t, j] = sum_s gates[t, s] * y[t*top_k + s, j]
 * accumulated with f32 fma from +0 in ascending s.
 * y device f32 [m*top_k, n]; gates device f32 [m, top_k]; out device f32
 * [m, n] (must not overlap y).
 */
int eidm_combine(uint32_t m, uint32_t top_k, uint32_t n, const float* y, const float* gates,
                 float* out, void* stream);

/*
 * Device-side check of an id table before it is used (mlx-native
 * dense_matmul_id_auto.rs: the shape key's id multiplicity,
 * DenseMatmulIdMultiplicity; distinct-per-token profile ids in
 * fn calibration_buffers).  An entry r = t*top_k + s is bad when
 * ids[r] >= n_experts or, with EIDM_IDS_DISTINCT_PER_TOKEN, when it equals
 * an earlier slot of token t.
 * ids           device u32 [m, top_k]
 * multiplicity  eidm_multiplicity of the table
 * bad_index_out host int32*: the smallest bad r, or -1 when none
 * Returns EIDM_OK when every entry is good and EIDM_E_IDS otherwise.
 * Synchronous: it waits for `stream` (so it cannot be captured in a graph).
 * Calls on one device share a device word: calls from several host threads
 * at once are serialised inside the library.  Requires m*top_k < 2^31.
 */
int eidm_validate_ids(const uint32_t* ids, uint32_t m, uint32_t top_k, uint32_t n_experts,
                      int multiplicity, int32_t* bad_index_out, void* stream);

/*
 * The whole path in one call: route (eidm_route_topk) -> matmul
 * (eidm_matmul_id) -> combine (eidm_combine), enqueued in order on
 * `stream`.  logits device f32 [m, n_experts]; bias device f32
 * [n_experts] or NULL; ids/gates/y/out are caller buffers that receive the
 * intermediate and final results.  shape->id_multiplicity must be
 * DISTINCT_PER_TOKEN (the router's ids are distinct).
 * When the route taken is Direct and top_k <= 16, the three steps run as
 * one kernel (per token and column group: route, Direct product of every
 * slot, combine) with the same results bit for bit as the three separate
 * calls; ids, gates and y are still written.
 */
int eidm_moe_forward(const eidm_shape* shape, int route, const void* weights,
                     uint64_t weight_bytes, const float* input, const float* logits,
                     const float* bias, int renormalize, uint32_t* ids, float* gates, float* y,
                     float* out, void* scratch, uint64_t scratch_bytes, void* stream,
                     int* route_taken);

/*
 * The mixture-of-experts expert FFN over routed rows (hf2q
 * dense_ffn_arena.rs MoeFfnArena: ids/weights [seq*topk], gate_all, up_all,
 * h_all [total_rows, m_moe] f32, y_all [total_rows, h], weighted reduce;
 * cortiq-engine mimo_moe.rs bank_tests: sum over picks of
 * w * down(silu(gate.x) (*) up.x)):
 *   ids, gates = route(logits, bias)                 (eidm_route_topk)
 *   g = matmul_id(W_gate, x), u = matmul_id(W_up, x) (shared layout, n = inter, k = hidden)
 *   h = silu(g) * u, silu(v) = v / (1 + exp(-v))      (f32, in place over g)
 *   y = matmul_id(W_down, h)                         (slotted layout, n = hidden, k = inter)
 *   out = combine(y, gates)                          (eidm_combine)
 * W_gate and W_up are [n_experts][inter][hidden] at gate_up_stride_bytes
 * per expert (one extent, gate_up_bytes, vouched for both); W_down is
 * [n_experts][hidden][inter] at down_stride_bytes.  x device f32
 * [m, hidden]; logits device f32 [m, n_experts]; bias device f32
 * [n_experts] or NULL; ids u32 / gates f32 [m, top_k] and out f32
 * [m, hidden] receive results; scratch device, 256-byte aligned, at least
 * eidm_moe_ffn_scratch_bytes(shape) bytes (intermediates, Grouped scratch).
 * `route` (AUTO, DIRECT, GROUPED) applies to the three projections alike;
 * route_taken (optional) receives the route that ran.  The router's limits
 * apply (top_k <= min(n_experts, 64), n_experts <= 2048).
 */
typedef struct eidm_ffn_shape {
    uint32_t struct_size;          /* sizeof(eidm_ffn_shape) */
    int32_t weight_dtype;          /* eidm_dtype of all three weights */
    uint32_t m, hidden, inter, top_k, n_experts, reserved0;
    uint64_t gate_up_stride_bytes; /* bytes between experts of W_gate and of W_up */
    uint64_t down_stride_bytes;    /* bytes between experts of W_down */
} eidm_ffn_shape;

/* Host-only: scratch bytes eidm_moe_ffn needs (0 if the shape is invalid). */
uint64_t eidm_moe_ffn_scratch_bytes(const eidm_ffn_shape* shape);

int eidm_moe_ffn(const eidm_ffn_shape* shape, int route, const void* w_gate, const void* w_up,
                 uint64_t gate_up_bytes, const void* w_down, uint64_t down_bytes, const float* x,
                 const float* logits, const float* bias, int renormalize, uint32_t* ids, float* gates,
                 float* out, void* scratch, uint64_t scratch_bytes, void* stream, int* route_taken);

/*
 * Activation-time route calibration and the frozen plan (mlx-native
 * dense_matmul_id_auto.rs: fn calibration_buffers, fn calibrate_one_inner
 * and its winner rule, fn resolve_dense_matmul_id_auto_route).
 *
 * eidm_calibrate takes, for one exact shape and the caller's weights, a
 * shape Grouped cannot run straight to Direct (no GPU work).  Otherwise it
 * runs, on each of two routing profiles with the page's adversarial
 * activations -- DISTINCT_PER_TOKEN shapes: balanced ids (t+s) mod n_experts
 * and skewed ids s; MAY_REPEAT shapes: ids t mod n_experts for both --
 *   1. a Direct proof and a Grouped proof on poisoned outputs with a guard:
 *      every output must be overwritten with a finite value, the guard
 *      untouched, and Grouped's bits equal to Direct's;
 *   2. five timing rounds, alternating which form runs first; each call is
 *      timed by the host clock around launch + synchronisation (wall) and by
 *      HIP events on `stream` (GPU).
 * Grouped is chosen only if, on both profiles, its median wall time is at
 * most 0.95 x Direct's, its 75th-percentile wall time is below Direct's
 * 25th percentile and its median GPU time is at most 1.02 x Direct's
 * (percentiles of 5 sorted samples v: v[1], v[2], v[3]).  A failed Direct
 * proof aborts (EIDM_E_DEVICE); any Grouped failure or difference keeps
 * Direct.  The decision is stored in the plan for the exact shape.
 *
 * Activation limits (DenseMatmulIdCalibrationLimits, fail-closed): a plan
 * counts, from eidm_plan_create (or eidm_plan_set_limits) on, the elapsed
 * time, the distinct shapes calibrated (cases) and the host waits on the GPU
 * (submissions: 1 for the inputs, then per profile 3 for the proofs and 10
 * for the timing samples; 27 for a shape Grouped can run).  Calibrating a
 * new shape beyond max_cases fails (EIDM_E_INVALID, nothing stored).  A
 * shape whose complete gate the remaining submissions cannot cover, or that
 * starts after the deadline, takes Direct without GPU work; a deadline that
 * passes during the proofs or timing, or before the route is chosen, also
 * gives Direct (reason EIDM_CAL_BUDGET).  eidm_plan_freeze after the
 * deadline turns every Grouped entry of the plan into Direct.
 * Synchronous; not capturable in a graph; the workspace belongs to the call.
 */
typedef struct eidm_plan eidm_plan; /* opaque; host memory owned by the library */

typedef enum eidm_calibration_reason {
    EIDM_CAL_GROUPED_WINS = 0,      /* every test passed: Grouped */
    EIDM_CAL_GROUPED_NOT_LEGAL = 1, /* Grouped cannot run this shape */
    EIDM_CAL_GROUPED_FAILED = 2,    /* a Grouped call failed or left outputs unwritten */
    EIDM_CAL_NOT_IDENTICAL = 3,     /* Grouped's bits differ from Direct's */
    EIDM_CAL_WALL_MEDIAN = 4,       /* median wall time above 0.95 x Direct's */
    EIDM_CAL_WALL_QUARTILES = 5,    /* 75th-percentile wall not below Direct's 25th */
    EIDM_CAL_GPU_MEDIAN = 6,        /* median GPU time above 1.02 x Direct's */
    EIDM_CAL_BUDGET = 7             /* the activation limits left no complete gate */
} eidm_calibration_reason;

/* Activation limits of a plan; every field nonzero.  Defaults: 15000 ms,
 * 256 cases, 6145 submissions. */
typedef struct eidm_calibration_limits {
    uint32_t struct_size;     /* set to sizeof(eidm_calibration_limits) by the caller */
    uint32_t max_cases;       /* distinct shapes the plan may calibrate */
    uint32_t max_submissions; /* host waits on the GPU over all calibrations of the plan */
    uint32_t reserved0;
    uint64_t max_elapsed_ms;  /* wall time from the limits' start to eidm_plan_freeze */
} eidm_calibration_limits;

typedef struct eidm_calibration {
    uint32_t struct_size;  /* set to sizeof(eidm_calibration) by the caller */
    int32_t route;         /* the route stored for the shape */
    int32_t grouped_legal; /* Grouped could run the shape */
    int32_t bit_identical; /* Grouped reproduced Direct's bits on both profiles */
    int32_t reason;        /* eidm_calibration_reason */
    uint32_t submissions;  /* host waits on the GPU this call made */
    /* per profile (0 balanced, 1 skewed), microseconds over 5 samples;
     * the grouped_* fields are 0 when Grouped did not run */
    double direct_wall_p25[2], direct_wall_median[2], direct_wall_p75[2], direct_gpu_median[2];
    double grouped_wall_p25[2], grouped_wall_median[2], grouped_wall_p75[2], grouped_gpu_median[2];
} eidm_calibration;

/* A new empty plan (NULL when out of host memory); destroy with
 * eidm_plan_destroy.  A plan may be shared by threads. */
eidm_plan* eidm_plan_create(void);
void eidm_plan_destroy(eidm_plan* plan);

/* Replace the plan's activation limits and restart its clock; only before
 * its first eidm_calibrate (else EIDM_E_INVALID, as for a zero limit). */
int eidm_plan_set_limits(eidm_plan* plan, const eidm_calibration_limits* limits);

/* Host-only: device workspace bytes eidm_calibrate needs for the shape (0 if
 * the shape is invalid).  The workspace must be 256-byte aligned. */
uint64_t eidm_calibration_workspace_bytes(const eidm_shape* shape);

/* Calibrate one exact shape on the caller's weights (device, as in
 * eidm_matmul_id).  workspace: device, eidm_calibration_workspace_bytes.
 * receipt: host, struct_size set; receives the measurements and decision.
 * Fails with EIDM_E_INVALID on a frozen plan. */
int eidm_calibrate(eidm_plan* plan, const eidm_shape* shape, const void* weights, uint64_t weight_bytes,
                   void* workspace, uint64_t workspace_bytes, void* stream, eidm_calibration* receipt);

/* No further calibration; lookups keep working.  After the activation
 * deadline every Grouped entry becomes Direct first.  downgraded (may be
 * NULL) receives how many entries that changed. */
int eidm_plan_freeze(eidm_plan* plan, uint32_t* downgraded);

/* Host-only lookup: an exact calibrated shape gives its stored route; a
 * shape equal to a calibrated one in everything but m gives Direct;
 * anything else is EIDM_E_UNSUPPORTED. */
int eidm_plan_route(const eidm_plan* plan, const eidm_shape* shape, int* route);

/* eidm_matmul_id with the route from eidm_plan_route; fails before any work
 * is enqueued when the plan has no route for the shape. */
int eidm_matmul_id_planned(const eidm_plan* plan, const eidm_shape* shape, const void* weights,
                           uint64_t weight_bytes, const float* input, const uint32_t* ids, float* output,
                           void* scratch, uint64_t scratch_bytes, void* stream, int* route_taken);

#ifdef __cplusplus
}
#endif

#endif /* EIDM_H */
