/*
 * eidm_oracle.c -- plain, slow CPU oracle for the expert-ID matmul path.
 *
 * TEST INFRASTRUCTURE ONLY.  Nothing in the product path may link, load or
 * call this file: only the tests, the smoke check and the CPU-baseline leg of
 * the benchmark use it.  It shares no source, header, table or constant with
 * the HIP library; it is written from the pages' statement of what is
 * computed, as directly as possible, in double precision.
 *
 * Pages cited (docs.rs source views):
 *   [auto]  mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs
 *   [mimo]  cortiq-engine 0.7.7, src/mimo_moe.rs
 *   [arena] hf2q, src/inference/models/qwen35/dense_ffn_arena.rs
 *   [eagle] hf2q 0.1.1, src/inference/spec_decode/eagle3/forward.rs
 *
 * Every function here is pinned by a CPU test against something other than
 * itself (brute force in numpy, closed forms, invariants, the pages' worked
 * example); the pin of each is named in its comment.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

enum { OR_F32 = 0, OR_F16 = 1, OR_BF16 = 2 };
enum { OR_SHARED_PER_TOKEN = 0, OR_SLOTTED = 1 };

static int dtype_size(int dtype) {
    switch (dtype) {
    case OR_F32: return 4;
    case OR_F16: return 2;
    case OR_BF16: return 2;
    default: return 0;
    }
}

/*
 * Native weight scalar -> real value, exactly ([auto], the value-independence
 * theorem statement: both routes widen each native weight scalar to f32
 * before the f32 multiply-add; the widening is exact for all three types).
 *   f32:  the IEEE binary32 value of the 4 bytes.
 *   bf16: the upper half of a binary32 (value of bits << 16).
 *   f16:  IEEE binary16, decoded from its definition: sign, 5-bit biased
 *         exponent (bias 15), 10-bit fraction; exponent 0 is subnormal
 *         (fraction * 2^-24), exponent 31 is inf/NaN.
 * Pin: exhaustive over all 65536 bf16 and f16 patterns against numpy's own
 * conversions.
 */
double oracle_widen(int dtype, const void* p) {
    if (dtype == OR_F32) {
        float f;
        memcpy(&f, p, 4);
        return (double)f;
    }
    uint16_t h;
    memcpy(&h, p, 2);
    if (dtype == OR_BF16) {
        uint32_t bits = (uint32_t)h << 16;
        float f;
        memcpy(&f, &bits, 4);
        return (double)f;
    }
    /* binary16 */
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1f;
    int frac = h & 0x3ff;
    double v;
    if (expo == 0) {
        v = ldexp((double)frac, -24);
    } else if (expo == 31) {
        v = frac ? NAN : INFINITY;
    } else {
        v = ldexp(1.0 + frac / 1024.0, expo - 15);
    }
    return sign ? -v : v;
}

/*
 * Bytes a weight buffer must span: the last expert starts at
 * (n_experts-1)*stride and holds n*k scalars ([auto], fn validate_cases:
 * the weight extent must reach the capability's required bytes; worked
 * example in the test cached_grouped_a_b_a_...: f32, n=5, k=7, 4 experts,
 * stride 152 B, a 596-byte buffer).  Returns 0 on overflow or bad dtype.
 * Pin: the 596-byte example and the padded 832-byte bf16 stride of the
 * page's test_shape.
 */
uint64_t oracle_required_weight_bytes(int dtype, uint32_t n, uint32_t k,
                                      uint32_t n_experts, uint64_t stride) {
    int size = dtype_size(dtype);
    if (!size || n_experts == 0) return 0;
    unsigned __int128 body = (unsigned __int128)n * k * (unsigned)size;
    unsigned __int128 total = (unsigned __int128)(n_experts - 1) * stride + body;
    if (total >> 64) return 0;
    return (uint64_t)total;
}

/*
 * Router ([mimo] module doc: each token picks 8 of 256 experts by a sigmoid
 * score plus a per-expert selection bias; bank_tests arch(): router_sigmoid
 * and norm_topk_prob both true, tensors mlp.gate.weight and mlp.expert_bias;
 * Dynamic::run: each pick's final weight is p[e] / wsum, applied with
 * route_scale 1.0).
 *
 *   s[t,e]   = sigmoid(logit[t,e]) = 1 / (1 + e^-logit), rounded to f32
 *   sel[t,e] = s[t,e] + bias[e]   (one f32 addition; bias only selects)
 *   ids[t,:] = the top_k experts by sel, largest first; equal sel -> lower
 *              expert index first
 *   gate     = s[t,id] / sum over the picks of s (renormalize != 0),
 *              or s[t,id] itself (renormalize == 0)
 *
 * The selection is an integer decided by floating point, so it is taken in
 * f32 like the kernel's: sigmoid is evaluated in double and rounded once to
 * f32 (the correctly rounded value, up to the double evaluation's error),
 * and the biased key is one f32 add.  Gates are reported in double.
 * Logits must be finite (returns -1 otherwise).
 * Pins: bias = 0 -> ids equal a plain argsort of the logits (sigmoid is
 * monotone); brute-force full sort in numpy; sigmoid(0) = 1/2 exactly;
 * renormalized gates sum to 1.
 */
int oracle_route(const float* logits, const float* bias, uint32_t m, uint32_t n_experts,
                 uint32_t top_k, int renormalize, uint32_t* ids, double* gates,
                 float* sigma_out, float* sel_out) {
    if (top_k == 0 || top_k > n_experts) return -1;
    float* s = (float*)malloc(sizeof(float) * n_experts);
    float* sel = (float*)malloc(sizeof(float) * n_experts);
    char* taken = (char*)malloc(n_experts);
    if (!s || !sel || !taken) {
        free(s); free(sel); free(taken);
        return -2;
    }
    int rc = 0;
    for (uint32_t t = 0; t < m && rc == 0; ++t) {
        for (uint32_t e = 0; e < n_experts; ++e) {
            float lg = logits[(size_t)t * n_experts + e];
            if (!isfinite(lg)) { rc = -1; break; }
            double sd = 1.0 / (1.0 + exp(-(double)lg));
            s[e] = (float)sd;
            float b = bias ? bias[e] : 0.0f;
            volatile float add = s[e] + b; /* a single f32 rounding */
            sel[e] = add;
            taken[e] = 0;
            if (sigma_out) sigma_out[(size_t)t * n_experts + e] = s[e];
            if (sel_out) sel_out[(size_t)t * n_experts + e] = sel[e];
        }
        if (rc) break;
        double wsum = 0.0;
        for (uint32_t j = 0; j < top_k; ++j) {
            int best = -1;
            for (uint32_t e = 0; e < n_experts; ++e) {
                if (taken[e]) continue;
                /* strictly greater: an equal key keeps the lower index */
                if (best < 0 || sel[e] > sel[best]) best = (int)e;
            }
            taken[best] = 1;
            ids[(size_t)t * top_k + j] = (uint32_t)best;
            wsum += (double)s[best];
        }
        for (uint32_t j = 0; j < top_k; ++j) {
            uint32_t e = ids[(size_t)t * top_k + j];
            gates[(size_t)t * top_k + j] = renormalize ? (double)s[e] / wsum : (double)s[e];
        }
    }
    free(s); free(sel); free(taken);
    return rc;
}

/*
 * One output of the expert-ID matmul for routed row r = t*top_k + slot
 * ([auto] module doc and value-independence theorem: input addressing,
 * expert base, weight scalar index, widening, multiply-add; fn
 * calibration_buffers: the input has m rows when shared per token and
 * m*top_k rows when slotted; ids are [m, top_k], routed-row major):
 *
 *   y[r, j] = sum_c W_e[j, c] * x_row(r)[c],   e = ids[r]
 *   W_e[j, c] at byte  e*expert_stride + (j*k + c)*sizeof(dtype)
 *   x_row(r) = x[r / top_k] (shared per token) or x[r] (slotted)
 *
 * Each product of a widened weight and an f32 activation is exact in double
 * (at most 24+24 significant bits); the sum is accumulated in double and is
 * returned unrounded.  An id >= n_experts has no weights: the output is NaN.
 */
static double one_output(int dtype, uint32_t n, uint32_t k, uint32_t top_k,
                         uint32_t n_experts, uint64_t stride, int layout,
                         const uint8_t* w, const float* x, const uint32_t* ids,
                         uint64_t r, uint32_t j) {
    uint32_t e = ids[r];
    if (e >= n_experts) return NAN;
    int size = dtype_size(dtype);
    const float* xr = layout == OR_SLOTTED ? x + r * k : x + (r / top_k) * k;
    const uint8_t* wrow = w + (uint64_t)e * stride + (uint64_t)j * k * size;
    double acc = 0.0;
    for (uint32_t c = 0; c < k; ++c) acc += oracle_widen(dtype, wrow + (uint64_t)c * size) * (double)xr[c];
    return acc;
}

/*
 * Full y [m*top_k, n] in double.  Pins: numpy float64 brute force on small
 * shapes (including the pages' tail shapes); top_k = 1 with one expert ->
 * numpy x @ W.T; identity expert (n = k, W = I) -> y == x exactly; a row
 * permutation permutes y; moving an expert to another index/stride and
 * remapping ids leaves y unchanged.
 */
int oracle_matmul_id(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                     uint32_t n_experts, uint64_t stride, int layout, const void* weights,
                     const float* x, const uint32_t* ids, double* y) {
    if (!dtype_size(dtype) || m == 0 || n == 0 || k == 0 || top_k == 0 || n_experts == 0) return -1;
    uint64_t rows = (uint64_t)m * top_k;
    for (uint64_t r = 0; r < rows; ++r)
        for (uint32_t j = 0; j < n; ++j)
            y[r * n + j] = one_output(dtype, n, k, top_k, n_experts, stride, layout,
                                      (const uint8_t*)weights, x, ids, r, j);
    return 0;
}

/*
 * oracle_matmul_id on `threads` host threads: the outputs (routed row,
 * column), numbered r*n + j, are split into `threads` contiguous ranges and
 * each thread evaluates its range with the same per-output routine.  The
 * values are those of oracle_matmul_id bit for bit (each output is computed
 * the same way, by one thread).  Used for the host-core baseline and for
 * full-size checks; pin: equality with oracle_matmul_id.
 */
typedef struct {
    int dtype;
    uint32_t n, k, top_k, n_experts;
    uint64_t stride;
    int layout;
    const uint8_t* w;
    const float* x;
    const uint32_t* ids;
    double* y;
    uint64_t begin, end;
} mm_part;

static void* mm_worker(void* arg) {
    const mm_part* p = (const mm_part*)arg;
    for (uint64_t o = p->begin; o < p->end; ++o) {
        const uint64_t r = o / p->n;
        const uint32_t j = (uint32_t)(o % p->n);
        p->y[o] = one_output(p->dtype, p->n, p->k, p->top_k, p->n_experts, p->stride, p->layout, p->w, p->x,
                             p->ids, r, j);
    }
    return NULL;
}

int oracle_matmul_id_threads(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                             uint32_t n_experts, uint64_t stride, int layout, const void* weights,
                             const float* x, const uint32_t* ids, double* y, int threads) {
    if (!dtype_size(dtype) || m == 0 || n == 0 || k == 0 || top_k == 0 || n_experts == 0) return -1;
    if (threads < 1 || threads > 1024) return -1;
    const uint64_t total = (uint64_t)m * top_k * n;
    mm_part* parts = (mm_part*)calloc((size_t)threads, sizeof(mm_part));
    pthread_t* tids = (pthread_t*)calloc((size_t)threads, sizeof(pthread_t));
    if (!parts || !tids) {
        free(parts);
        free(tids);
        return -2;
    }
    int started = 0, rc = 0;
    for (int t = 0; t < threads; ++t) {
        mm_part* p = &parts[t];
        p->dtype = dtype;
        p->n = n;
        p->k = k;
        p->top_k = top_k;
        p->n_experts = n_experts;
        p->stride = stride;
        p->layout = layout;
        p->w = (const uint8_t*)weights;
        p->x = x;
        p->ids = ids;
        p->y = y;
        p->begin = total * (uint64_t)t / (uint64_t)threads;
        p->end = total * (uint64_t)(t + 1) / (uint64_t)threads;
        if (pthread_create(&tids[t], NULL, mm_worker, p) != 0) {
            rc = -3;
            break;
        }
        ++started;
    }
    for (int t = 0; t < started; ++t) pthread_join(tids[t], NULL);
    free(parts);
    free(tids);
    return rc;
}

/*
 * The same outputs at chosen (row, column) pairs only, for spot checks of
 * full-size problems: out[i] = y[rows[i], cols[i]].
 */
int oracle_matmul_id_at(int dtype, uint32_t m, uint32_t n, uint32_t k, uint32_t top_k,
                        uint32_t n_experts, uint64_t stride, int layout, const void* weights,
                        const float* x, const uint32_t* ids, uint64_t count,
                        const uint64_t* rows, const uint32_t* cols, double* out) {
    if (!dtype_size(dtype) || m == 0 || n == 0 || k == 0 || top_k == 0 || n_experts == 0) return -1;
    for (uint64_t i = 0; i < count; ++i) {
        if (rows[i] >= (uint64_t)m * top_k || cols[i] >= n) return -1;
        out[i] = one_output(dtype, n, k, top_k, n_experts, stride, layout,
                            (const uint8_t*)weights, x, ids, rows[i], cols[i]);
    }
    return 0;
}

/*
 * Gate-weighted sum over the top_k slots of each token ([mimo] Dynamic::run
 * and run_rows: every pick's expert output is scaled by its final weight and
 * the picks are summed; [arena] MoeFfnArena: ids and weights are
 * [seq*topk], y_all is [seq*topk, h], and the weighted reduce writes
 * [seq, h]):
 *
 *   out[t, j] = sum_s gate[t, s] * y[t*top_k + s, j]
 *
 * in double.  Pin: one-hot gates select one y row exactly; numpy einsum.
 */
int oracle_combine(uint32_t m, uint32_t top_k, uint32_t n, const double* y,
                   const double* gates, double* out) {
    for (uint64_t t = 0; t < m; ++t)
        for (uint32_t j = 0; j < n; ++j) {
            double acc = 0.0;
            for (uint32_t s = 0; s < top_k; ++s)
                acc += gates[t * top_k + s] * y[(t * top_k + s) * n + j];
            out[t * n + j] = acc;
        }
    return 0;
}

/*
 * Id -> row map used by the grouped form ([auto] fn expected_dispatches:
 * the grouped route first runs a map pass over the ids that builds per-expert
 * row lists, then tiles each expert's rows; its scratch is sized by
 * n_experts and m).  Definition: a stable counting sort of the routed rows
 * r = 0 .. m*top_k-1 by key min(ids[r], n_experts), so bucket n_experts
 * collects ids that name no expert.
 *   counts[b]  = number of rows with key b            (b = 0 .. n_experts)
 *   offsets[b] = sum of counts[b'] for b' < b          (b = 0 .. n_experts+1)
 *   rows[offsets[b] ..] = the rows with key b, ascending
 * Pins: closed forms of the balanced ((t+s) mod E: every expert gets
 * m*top_k/E rows) and maximally skewed (id = s: experts 0..top_k-1 get m
 * rows, the rest none) profiles; numpy stable argsort.
 */
int oracle_map(const uint32_t* ids, uint64_t rows_total, uint32_t n_experts,
               uint32_t* counts, uint32_t* offsets, uint32_t* rows) {
    for (uint32_t b = 0; b <= n_experts; ++b) counts[b] = 0;
    for (uint64_t r = 0; r < rows_total; ++r) {
        uint32_t key = ids[r] < n_experts ? ids[r] : n_experts;
        counts[key]++;
    }
    offsets[0] = 0;
    for (uint32_t b = 0; b <= n_experts; ++b) offsets[b + 1] = offsets[b] + counts[b];
    uint64_t out = 0;
    for (uint32_t b = 0; b <= n_experts; ++b)
        for (uint64_t r = 0; r < rows_total; ++r) {
            uint32_t key = ids[r] < n_experts ? ids[r] : n_experts;
            if (key == b) rows[out++] = (uint32_t)r;
        }
    return 0;
}

/*
 * The mixture-of-experts expert FFN over routed rows ([mimo] bank_tests:
 * the exact reference output is the sum over picks of w * down(silu(gate.x)
 * (*) up.x), in f64; [arena] MoeFfnArena: gate_all and up_all come from a
 * shared-layout matmul_id over the token rows, h_all = silu(gate) * up, y_all
 * from a slotted-layout matmul_id over h_all, then the weighted reduce):
 *
 *   g[r, j] = sum_c Wg_e[j, c] x[t, c]      (j < inter, c < hidden)
 *   u[r, j] = sum_c Wu_e[j, c] x[t, c]
 *   h[r, j] = silu(g[r, j]) * u[r, j],   silu(v) = v / (1 + exp(-v))
 *   y[r, i] = sum_j Wd_e[i, j] h[r, j]      (i < hidden)
 *   out[t, i] = sum_s gates[t, s] y[t*top_k + s, i]
 * with e = ids[r], r = t*top_k + s; Wg, Wu are [E][inter][hidden] at
 * gu_stride bytes per expert, Wd is [E][hidden][inter] at down_stride.
 * Everything in double.  Pins: numpy float64 brute force on tiny shapes;
 * silu's odd-part identity silu(v) - silu(-v) = v; W_up = 0 gives 0;
 * doubling W_down doubles out exactly; the composition of oracle_matmul_id
 * (gate, up) and oracle_combine with an identity down projection.
 */
static double silu_d(double v) { return v / (1.0 + exp(-v)); }

int oracle_moe_ffn(int dtype, uint32_t m, uint32_t hidden, uint32_t inter, uint32_t top_k,
                   uint32_t n_experts, uint64_t gu_stride, uint64_t down_stride,
                   const void* w_gate, const void* w_up, const void* w_down, const float* x,
                   const uint32_t* ids, const double* gates, double* h_out, double* out) {
    int size = dtype_size(dtype);
    if (!size || !m || !hidden || !inter || !top_k || !n_experts) return -1;
    double* h = (double*)malloc(sizeof(double) * inter);
    if (!h) return -2;
    for (uint64_t t = 0; t < m; ++t)
        for (uint32_t i = 0; i < hidden; ++i) out[t * hidden + i] = 0.0;
    for (uint64_t t = 0; t < m; ++t)
        for (uint32_t s = 0; s < top_k; ++s) {
            uint64_t r = t * top_k + s;
            uint32_t e = ids[r];
            if (e >= n_experts) {
                free(h);
                return -3;
            }
            const float* xr = x + t * hidden;
            const uint8_t* wg = (const uint8_t*)w_gate + (uint64_t)e * gu_stride;
            const uint8_t* wu = (const uint8_t*)w_up + (uint64_t)e * gu_stride;
            for (uint32_t j = 0; j < inter; ++j) {
                double g = 0.0, u = 0.0;
                for (uint32_t c = 0; c < hidden; ++c) {
                    uint64_t off = ((uint64_t)j * hidden + c) * size;
                    g += oracle_widen(dtype, wg + off) * (double)xr[c];
                    u += oracle_widen(dtype, wu + off) * (double)xr[c];
                }
                h[j] = silu_d(g) * u;
                if (h_out) h_out[r * inter + j] = h[j];
            }
            const uint8_t* wd = (const uint8_t*)w_down + (uint64_t)e * down_stride;
            for (uint32_t i = 0; i < hidden; ++i) {
                double y = 0.0;
                for (uint32_t j = 0; j < inter; ++j)
                    y += oracle_widen(dtype, wd + ((uint64_t)i * inter + j) * size) * h[j];
                out[t * hidden + i] += gates[r] * y;
            }
        }
    free(h);
    return 0;
}
