// matmul_split16.hip -- the expert-ID matmul in the split-16 arithmetic:
// 16-bit weights kept exact in their own type, each f32 activation split
// exactly into three parts of that type, the products on the 16-bit matrix
// core (v_mfma_f32_16x16x32_bf16 / _f16).
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: the value-independence
// theorem statement asks the Grouped route to reproduce the Direct route's
// bits, differing only in which independent rows are computed together.
// Here both routes issue, per output, the same instruction sequence on the
// same operands; the instruction's result for an output does not depend on
// the row or column position it occupies in the 16 x 16 tile (checked on
// MI355X: equal rows and columns give equal results at all 256 positions,
// and one live row gives the same bits at every row), so the rows a tile
// carries beside an output do not change it.
//
// The order, per output (r, j), over steps of 32 k (zero past k; the step
// count rounded up to a multiple of 4):
//   hi: the p1 products of steps 4q .. 4q+3 in one chain from +0;
//       total = total + hi after every 4 steps (f32 add, total from +0);
//   lo: one chain from +0 over all steps, the p2 then the p3 products;
//   y = total + lo.
// Operand layout of one instruction (16 x 16 x 32): lane l supplies row or
// column l % 16 with k elements 8*(l/16) .. 8*(l/16)+7 of the step; result
// register v of lane l is row 4*(l/16) + v, column l % 16.
//
// The activations are split once per call into a scratch buffer: chunk c of
// 8 consecutive input elements becomes three 16-byte groups (p1, p2, p3).
#include <atomic>

#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

typedef __bf16 s16_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 s16_f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int s16u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSplitChunkHalves = 24;  // 16-bit elements per split chunk (3 parts x 8)
constexpr int kStepsPerRound = 4;      // steps of 32 k between hi restarts

template <int DT>
__device__ __forceinline__ f32x4 s16_mfma(const s16u32x4& a, const s16u32x4& b, f32x4 c) {
    if constexpr (DT == kDtypeF16)
        return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(s16_f16x8, a),
                                                      __builtin_bit_cast(s16_f16x8, b), c, 0, 0, 0);
    else
        return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(s16_bf16x8, a),
                                                       __builtin_bit_cast(s16_bf16x8, b), c, 0, 0, 0);
}

// f32 -> 16-bit, round to nearest even; the value back in f32
template <int DT> __device__ __forceinline__ uint32_t s16_round(float v);
template <> __device__ __forceinline__ uint32_t s16_round<kDtypeBF16>(float v) {
    const uint32_t u = __float_as_uint(v);
    if ((u & 0x7f800000u) == 0x7f800000u) return (u >> 16) | ((u & 0xffffu) ? 0x40u : 0u);  // inf, NaN stay
    return (u + 0x7fffu + ((u >> 16) & 1u)) >> 16;
}
template <> __device__ __forceinline__ uint32_t s16_round<kDtypeF16>(float v) {
    return (uint32_t)__builtin_bit_cast(uint16_t, (_Float16)v);
}
template <int DT> __device__ __forceinline__ float s16_value(uint32_t h);
template <> __device__ __forceinline__ float s16_value<kDtypeBF16>(uint32_t h) { return __uint_as_float(h << 16); }
template <> __device__ __forceinline__ float s16_value<kDtypeF16>(uint32_t h) {
    return (float)__builtin_bit_cast(_Float16, (uint16_t)h);
}

// x = p1 + p2 + p3: p1 = rn(x), p2 = rn(x - p1), p3 = rn(x - p1 - p2); the
// differences are exact in f32.  A non-finite x keeps p1 = rn(x), p2 = p3 = 0.
template <int DT>
__device__ __forceinline__ void s16_split(float v, uint32_t& p1, uint32_t& p2, uint32_t& p3) {
    p1 = s16_round<DT>(v);
    const float f1 = s16_value<DT>(p1);
    if (!__builtin_isfinite(v) || !__builtin_isfinite(f1)) {
        p2 = p3 = 0;
        return;
    }
    const float r1 = v - f1;
    p2 = s16_round<DT>(r1);
    const float r2 = r1 - s16_value<DT>(p2);
    p3 = s16_round<DT>(r2);
}

template <int DT>
__global__ __launch_bounds__(256) void split_x_kernel(const float* __restrict__ x, uint64_t chunks,
                                                      uint16_t* __restrict__ xs) {
    for (uint64_t c = (uint64_t)blockIdx.x * blockDim.x + threadIdx.x; c < chunks;
         c += (uint64_t)gridDim.x * blockDim.x) {
        const f32x4 a = reinterpret_cast<const f32x4*>(x)[2 * c];
        const f32x4 b = reinterpret_cast<const f32x4*>(x)[2 * c + 1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t p[3][8];
#pragma unroll
        for (int t = 0; t < 8; ++t) s16_split<DT>(v[t], p[0][t], p[1][t], p[2][t]);
        s16u32x4* out = reinterpret_cast<s16u32x4*>(xs + c * kSplitChunkHalves);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            out[q] = s16u32x4{p[q][0] | (p[q][1] << 16), p[q][2] | (p[q][3] << 16), p[q][4] | (p[q][5] << 16),
                              p[q][6] | (p[q][7] << 16)};
    }
}

// ---------------------------------------------------------------- Direct
// One wavefront per (routed row, 32 columns): the row is live in tile row 0
// (lanes 0, 16, 32, 48 supply its parts; the other rows are zero), two
// 16-column tiles.  Operands of a round (4 steps) are loaded one round ahead.
constexpr int kDs16Cols = 32;

template <int DT>
__global__ __launch_bounds__(64) void direct_split16_kernel(MatmulArgs a) {
    const uint32_t n = a.n, k = a.k, kc = a.k / 8;
    const uint32_t col_tiles = (n + kDs16Cols - 1) / kDs16Cols;
    const uint32_t r = blockIdx.x / col_tiles;
    const uint32_t c0 = (blockIdx.x - r * col_tiles) * kDs16Cols;
    const int l = threadIdx.x, l16 = l & 15, g = l >> 4;
    const uint32_t e = a.ids[r];
    float* yrow = a.output + (size_t)r * n;
    if (e >= a.n_experts) {  // no weights for this row: quiet NaN
        if (l < kDs16Cols && c0 + l < n) yrow[c0 + l] = quiet_nan();
        return;
    }
    const uint32_t xr = a.layout == 1 ? r : r / a.top_k;
    const uint16_t* xs = a.xsplit + (size_t)xr * kc * kSplitChunkHalves;
    const bool live = l16 == 0;
    const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;
    const uint8_t* wrow[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) {
        const uint32_t col = min(c0 + 16 * ct + l16, n - 1);
        wrow[ct] = wexp + (size_t)col * k * 2;
    }
    const uint32_t rounds = (k + 127) / 128;
    struct Ops {
        s16u32x4 x[kStepsPerRound][3];
        s16u32x4 w[kStepsPerRound][2];
    };
    auto load = [&](uint32_t q, Ops& o) {
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s) {
            const uint32_t ch = 16 * q + 4 * s + g;  // this lane's chunk of the step
            const bool in = ch < kc;
            const uint32_t cc = in ? ch : kc - 1;
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                s16u32x4 v = {0u, 0u, 0u, 0u};
                if (live) v = *reinterpret_cast<const s16u32x4*>(xs + (size_t)cc * kSplitChunkHalves + 8 * p);
                o.x[s][p] = in ? v : s16u32x4{0u, 0u, 0u, 0u};
            }
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const s16u32x4 v = *reinterpret_cast<const s16u32x4*>(wrow[ct] + (size_t)cc * 16);
                o.w[s][ct] = in ? v : s16u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    f32x4 tot[2], lo[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) tot[ct] = lo[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const Ops& o) {
        f32x4 hi[2];
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) hi[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                hi[ct] = s16_mfma<DT>(o.x[s][0], o.w[s][ct], hi[ct]);
                lo[ct] = s16_mfma<DT>(o.x[s][1], o.w[s][ct], lo[ct]);
                lo[ct] = s16_mfma<DT>(o.x[s][2], o.w[s][ct], lo[ct]);
            }
#pragma unroll
        for (int ct = 0; ct < 2; ++ct)
#pragma unroll
            for (int v = 0; v < 4; ++v) tot[ct][v] = tot[ct][v] + hi[ct][v];
    };
    // two register slots with static names, each refilled two rounds ahead
    Ops o0, o1;
    load(0, o0);
    if (rounds > 1) load(1, o1);
    for (uint32_t q = 0; q < rounds; q += 2) {
        compute(o0);
        if (q + 2 < rounds) load(q + 2, o0);
        if (q + 1 < rounds) {
            compute(o1);
            if (q + 3 < rounds) load(q + 3, o1);
        }
    }
    // tile row 0: register 0 of lanes 0..15
    if (g == 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint32_t col = c0 + 16 * ct + l16;
            if (col < n) yrow[col] = tot[ct][0] + lo[ct][0];
        }
    }
}

// ---------------------------------------------------------------- Grouped
// A job is 32 gathered rows of one expert (two 16-row tiles) by 128 output
// columns; a block of 4 wavefronts takes 32 columns each (two 16-column
// tiles).  Per round of 128 k the block stages the split activations of its
// 32 rows in LDS (double buffer); each wavefront's weights go straight into
// registers.  The rounds of all the jobs a block walks form one stream, its
// loads two rounds ahead.
constexpr int kGs16BM = 32;
constexpr int kGs16BN = 128;
constexpr int kGs16Waves = 4;
constexpr int kGs16Threads = 64 * kGs16Waves;
constexpr int kGs16RowBytes = 16 * 48 + 16;               // one row's 16 chunks of a round, padded
constexpr int kGs16Buf = kGs16BM * kGs16RowBytes;          // one round's activation tile
constexpr int kGs16Bufs = 3;
constexpr int kGs16Xcds = 8;

struct Gs16Job {
    uint32_t e, rc, col0, rbase;
};

template <int DT>
__global__ __launch_bounds__(kGs16Threads, 1) void grouped_split16_kernel(MatmulArgs a,
                                                                          const uint32_t* __restrict__ counts,
                                                                          const uint32_t* __restrict__ offsets,
                                                                          const uint32_t* __restrict__ rows) {
    const uint32_t buckets = a.n_experts + 1;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* xbuf = smem;                                                        // [3][32][784 B]
    uint32_t* job_start = reinterpret_cast<uint32_t*>(smem + kGs16Bufs * kGs16Buf);  // [buckets+1]
    uint32_t* cnt_s = job_start + buckets + 1;                                   // [buckets]
    uint32_t* off_s = cnt_s + buckets;                                           // [buckets]
    __shared__ uint32_t wave_tot[kGs16Waves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int l16 = lane & 15, g = lane >> 4;
    const uint32_t n = a.n, k = a.k, kc = a.k / 8;
    const uint32_t ntiles = (n + kGs16BN - 1) / kGs16BN;
    const uint32_t R = (k + 127) / 128;  // rounds per job

    // ---- job table: jobs per bucket -> exclusive prefix
    {
        const uint32_t per = (buckets + kGs16Threads - 1) / kGs16Threads;
        const uint32_t begin = min(buckets, (uint32_t)tid * per);
        const uint32_t end = min(buckets, begin + per);
        uint32_t s = 0;
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t c = counts[i];
            cnt_s[i] = c;
            off_s[i] = offsets[i];
            const uint32_t jobs = ((c + kGs16BM - 1) / kGs16BM) * ntiles;
            job_start[i] = jobs;
            s += jobs;
        }
        uint32_t inc = s;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d);
            if (lane >= d) inc += o;
        }
        if (lane == 63) wave_tot[wave] = inc;
        __syncthreads();
        uint32_t run = inc - s, total = 0;
        for (int w = 0; w < kGs16Waves; ++w) {
            if (w < wave) run += wave_tot[w];
            total += wave_tot[w];
        }
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t v = job_start[i];
            job_start[i] = run;
            run += v;
        }
        if (tid == 0) job_start[buckets] = total;
        __syncthreads();
    }
    const uint32_t total_jobs = job_start[buckets];
    // each XCD walks one contiguous share of the job list, its blocks side by
    // side (blocks are dealt to the XCDs round-robin)
    const uint32_t per_xcd = gridDim.x / kGs16Xcds;
    const uint32_t xcd_jobs = (total_jobs + kGs16Xcds - 1) / kGs16Xcds;
    const uint32_t xcd = blockIdx.x % kGs16Xcds;
    const uint32_t job0 = xcd * xcd_jobs + blockIdx.x / kGs16Xcds;
    const uint32_t job_end = min(total_jobs, (xcd + 1) * xcd_jobs);
    if (job0 >= job_end) return;  // the whole block leaves together
    const uint32_t my_jobs = (job_end - job0 + per_xcd - 1) / per_xcd;
    uint32_t top = 1;
    while (top * 2 <= buckets) top *= 2;
    auto decode = [&](uint32_t i) {  // block-uniform
        const uint32_t jb = job0 + i * per_xcd;
        uint32_t e = 0;
        for (uint32_t st = top; st; st >>= 1)
            if (e + st < buckets && job_start[e + st] <= jb) e += st;
        const uint32_t local = jb - job_start[e];
        const uint32_t mt = local / ntiles, nt = local - mt * ntiles;
        Gs16Job j;
        j.e = e;
        j.rc = min((uint32_t)kGs16BM, cnt_s[e] - mt * kGs16BM);
        j.col0 = nt * kGs16BN;
        j.rbase = off_s[e] + mt * kGs16BM;
        return j;
    };

    // ---- load side: the staging role of this thread (row tid/8, chunks
    // 2*(tid%8) and 2*(tid%8)+1 of a round) and this lane's weight rows
    const int srow = tid >> 3, schunk = 2 * (tid & 7);
    struct LoadJob {
        const uint16_t* xs;     // this thread's staged row, chunk 0
        const uint8_t* w[2];    // this lane's weight rows (two column tiles)
    };
    // the routed row this thread stages for job j (read one job ahead)
    auto stage_row = [&](const Gs16Job& j) { return rows[j.rbase + ((uint32_t)srow < j.rc ? (uint32_t)srow : 0u)]; };
    auto load_job = [&](const Gs16Job& j, uint32_t rr) {
        LoadJob L;
        const uint32_t xr = a.layout == 1 ? rr : rr / a.top_k;
        L.xs = a.xsplit + (size_t)xr * kc * kSplitChunkHalves;
        const uint32_t wexp = j.e < a.n_experts ? j.e : 0u;
        const uint8_t* base = static_cast<const uint8_t*>(a.weights) + (size_t)wexp * a.stride;
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint32_t col = min(j.col0 + 32 * wave + 16 * ct + l16, n - 1);
            L.w[ct] = base + (size_t)col * k * 2;
        }
        return L;
    };
    struct Stage {
        s16u32x4 x[2][3];       // two chunks x three parts
        s16u32x4 w[kStepsPerRound][2];
    };
    auto load_round = [&](const LoadJob& L, uint32_t q, Stage& st) {
#pragma unroll
        for (int c = 0; c < 2; ++c) {
            const uint32_t ch = 16 * q + schunk + c;
            const bool in = ch < kc;
            const uint32_t cc = in ? ch : kc - 1;
#pragma unroll
            for (int p = 0; p < 3; ++p) {
                const s16u32x4 v = *reinterpret_cast<const s16u32x4*>(L.xs + (size_t)cc * kSplitChunkHalves + 8 * p);
                st.x[c][p] = in ? v : s16u32x4{0u, 0u, 0u, 0u};
            }
        }
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s) {
            const uint32_t ch = 16 * q + 4 * s + g;
            const bool in = ch < kc;
            const uint32_t cc = in ? ch : kc - 1;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                const s16u32x4 v = *reinterpret_cast<const s16u32x4*>(L.w[ct] + (size_t)cc * 16);
                st.w[s][ct] = in ? v : s16u32x4{0u, 0u, 0u, 0u};
            }
        }
    };
    auto store_x = [&](int buf, const Stage& st) {
        uint8_t* dst = xbuf + buf * kGs16Buf + srow * kGs16RowBytes + schunk * 48;
#pragma unroll
        for (int c = 0; c < 2; ++c)
#pragma unroll
            for (int p = 0; p < 3; ++p) *reinterpret_cast<s16u32x4*>(dst + c * 48 + p * 16) = st.x[c][p];
    };

    // ---- compute side
    f32x4 tot[2][2], lo[2][2];
    auto compute_round = [&](int buf, const Stage& st) {
        f32x4 hi[2][2];
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) hi[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
        const uint8_t* src = xbuf + buf * kGs16Buf + l16 * kGs16RowBytes + g * 48;
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s) {
            s16u32x4 xa[2][3];
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int p = 0; p < 3; ++p)
                    xa[rt][p] = *reinterpret_cast<const s16u32x4*>(src + rt * 16 * kGs16RowBytes + s * 4 * 48 + p * 16);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    hi[rt][ct] = s16_mfma<DT>(xa[rt][0], st.w[s][ct], hi[rt][ct]);
                    lo[rt][ct] = s16_mfma<DT>(xa[rt][1], st.w[s][ct], lo[rt][ct]);
                    lo[rt][ct] = s16_mfma<DT>(xa[rt][2], st.w[s][ct], lo[rt][ct]);
                }
        }
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct)
#pragma unroll
                for (int v = 0; v < 4; ++v) tot[rt][ct][v] = tot[rt][ct][v] + hi[rt][ct][v];
    };
    // the output rows of this lane's results (read when the job starts)
    uint32_t yrows[2][4];
    auto read_yrows = [&](const Gs16Job& j) {
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t i = 16 * rt + 4 * g + v;
                yrows[rt][v] = rows[j.rbase + (i < j.rc ? i : 0u)];
            }
    };
    auto finish = [&](const Gs16Job& j) {
        const bool nan_rows = j.e == a.n_experts;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const uint32_t i = 16 * rt + 4 * g + v;  // row of the job
                if (i >= j.rc) continue;
                float* yrow = a.output + (size_t)yrows[rt][v] * n;
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) {
                    const uint32_t col = j.col0 + 32 * wave + 16 * ct + l16;
                    if (col < n) yrow[col] = nan_rows ? quiet_nan() : tot[rt][ct][v] + lo[rt][ct][v];
                }
            }
    };

    // The stream: position i = (job i / R, round i % R).  Position i is
    // computed from LDS buffer i % 3 and weight slot i % 3; its loads were
    // issued at position i - 2 and its activations stored to LDS at
    // position i - 1 (before that position's barrier).
    const uint32_t total_pos = my_jobs * R;
    Gs16Job jc = decode(0);             // job being computed
    read_yrows(jc);
    LoadJob Lj = load_job(jc, stage_row(jc));  // job being loaded
    uint32_t lj = 0, lq = 0;            // its job index and round
    uint32_t next_rr = my_jobs > 1 ? stage_row(decode(1)) : 0u;  // staged row of job lj + 1
    auto advance_load = [&]() {
        if (++lq == R) {
            lq = 0;
            if (++lj < my_jobs) {
                Lj = load_job(decode(lj), next_rr);
                if (lj + 1 < my_jobs) next_rr = stage_row(decode(lj + 1));
            }
        }
    };
    Stage ring0, ring1, ring2;  // register slots of positions i % 3 (static names: no indexed registers)
    load_round(Lj, lq, ring0);
    advance_load();
    if (total_pos > 1) {
        load_round(Lj, lq, ring1);
        advance_load();
    }
    store_x(0, ring0);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) tot[rt][ct] = lo[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t q = 0;  // round of the computed job
    uint32_t ci = 0;
    // Position i: compute from LDS buffer and register slot i % 3; load
    // position i + 2 into slot (i + 2) % 3; store position i + 1's staged
    // activations into LDS buffer (i + 1) % 3; one barrier.
    auto position = [&](uint32_t i, int buf, Stage& cur, Stage& nxt, Stage& ahead) __attribute__((always_inline)) {
        if (i + 2 < total_pos) {
            load_round(Lj, lq, ahead);
            advance_load();
        }
        compute_round(buf, cur);
        if (i + 1 < total_pos) store_x(buf == 2 ? 0 : buf + 1, nxt);
        if (++q == R) {
            finish(jc);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < 2; ++ct) tot[rt][ct] = lo[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
            q = 0;
            if (++ci < my_jobs) {
                jc = decode(ci);
                read_yrows(jc);
            }
        }
        __syncthreads();
    };
    for (uint32_t i = 0; i < total_pos; i += 3) {
        position(i, 0, ring0, ring1, ring2);
        if (i + 1 < total_pos) position(i + 1, 1, ring1, ring2, ring0);
        if (i + 2 < total_pos) position(i + 2, 2, ring2, ring0, ring1);
    }
}

}  // namespace

hipError_t launch_split16_x(const MatmulArgs& a, hipStream_t stream) {
    const uint64_t in_rows = a.layout == 1 ? (uint64_t)a.m * a.top_k : a.m;
    const uint64_t chunks = in_rows * (a.k / 8);
    uint64_t blocks = (chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks == 0) blocks = 1;
    if (a.dtype == kDtypeF16)
        hipLaunchKernelGGL(split_x_kernel<kDtypeF16>, dim3((uint32_t)blocks), dim3(256), 0, stream, a.input, chunks,
                           a.xsplit);
    else
        hipLaunchKernelGGL(split_x_kernel<kDtypeBF16>, dim3((uint32_t)blocks), dim3(256), 0, stream, a.input, chunks,
                           a.xsplit);
    return launched(EIDM_KERNEL_SPLIT_X, (uint32_t)blocks, 256, 0);
}

hipError_t launch_direct_split16(const MatmulArgs& a, hipStream_t stream) {
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t blocks = routed * ((a.n + kDs16Cols - 1) / kDs16Cols);
    if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
    if (a.dtype == kDtypeF16)
        hipLaunchKernelGGL(direct_split16_kernel<kDtypeF16>, dim3((uint32_t)blocks), dim3(64), 0, stream, a);
    else
        hipLaunchKernelGGL(direct_split16_kernel<kDtypeBF16>, dim3((uint32_t)blocks), dim3(64), 0, stream, a);
    return launched(EIDM_KERNEL_DIRECT_SPLIT16, (uint32_t)blocks, 64, 0);
}

hipError_t launch_grouped_split16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream) {
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t ntiles = (a.n + kGs16BN - 1) / kGs16BN;
    const uint64_t job_bound = (routed / kGs16BM + a.n_experts + 1) * ntiles;
    const size_t lds = (size_t)kGs16Bufs * kGs16Buf + (3 * (size_t)a.n_experts + 4) * sizeof(uint32_t);
    auto kernel = a.dtype == kDtypeF16 ? grouped_split16_kernel<kDtypeF16> : grouped_split16_kernel<kDtypeBF16>;
    static std::atomic<uint32_t> raised{0};
    const uint32_t bit = a.dtype == kDtypeF16 ? 1u : 2u;
    if (!(raised.load(std::memory_order_relaxed) & bit)) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        raised.fetch_or(bit, std::memory_order_relaxed);
    }
    const uint64_t resident = (uint64_t)(device_cus > 0 ? device_cus : 256);
    uint64_t grid = job_bound < resident ? job_bound : resident;
    grid = (grid + kGs16Xcds - 1) / kGs16Xcds * kGs16Xcds;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kGs16Threads), lds, stream, a, buf.counts, buf.offsets,
                       buf.rows);
    return launched(EIDM_KERNEL_GROUPED_SPLIT16, (uint32_t)grid, kGs16Threads, (uint32_t)lds);
}

}  // namespace eidm
