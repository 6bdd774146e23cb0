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
//   hi: one chain from +0 over all steps, the p1 products;
//   lo: one chain from +0 over all steps, the p2 then the p3 products;
//   y = hi + lo (one f32 add).
// Operand layout of one instruction (16 x 16 x 32): lane l supplies row or
// column l % 16 with k elements 8*(l/16) .. 8*(l/16)+7 of the step; result
// register v of lane l is row 4*(l/16) + v, column l % 16.
//
// The activations are split once per call into a scratch buffer: chunk c of
// 8 consecutive input elements becomes three 16-byte groups (p1, p2, p3).
// The buffer starts with a block of zeros, and each row is padded with zero
// chunks to a whole number of 128-k rounds, so no load needs a bounds test
// on its data: a load past k reads the zero block instead.
#include <atomic>

#include "eidm_device.hpp"
#include "eidm_internal.hpp"
#include "map_keyed.hpp"

namespace eidm {
namespace {

typedef __bf16 s16_bf16x8 __attribute__((ext_vector_type(8)));
typedef _Float16 s16_f16x8 __attribute__((ext_vector_type(8)));
typedef unsigned int s16u32x4 __attribute__((ext_vector_type(4)));

constexpr int kSplitChunkHalves = 24;  // 16-bit elements per split chunk (3 parts x 8)
constexpr int kStepsPerRound = 4;      // steps of 32 k per round (128 k)
constexpr int kZeroHalves = 128;       // the zero block at the start of the split buffer (256 bytes)

// split chunks per row: k/8 rounded up to a whole number of rounds (16 chunks)
__host__ __device__ inline uint32_t s16_row_chunks(uint32_t k) { return (k + 127) / 128 * 16; }

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

// xs: the zero block, then rows of s16_row_chunks(k) chunks (zero past k).
// Chunks t, t + stride, ... of the whole buffer for worker t of `stride`
// (worker 0 also writes the zero block).
template <int DT>
__device__ __forceinline__ void split_x_chunks(const float* __restrict__ x, uint32_t k, uint64_t rows,
                                               uint16_t* __restrict__ xs, uint64_t t, uint64_t stride) {
    const uint32_t kc = k / 8, kcp = s16_row_chunks(k);
    const uint64_t chunks = rows * kcp;
    if (t < kZeroHalves / 8) reinterpret_cast<s16u32x4*>(xs)[t] = s16u32x4{0u, 0u, 0u, 0u};
    uint16_t* body = xs + kZeroHalves;
    for (uint64_t c = t; c < chunks; c += stride) {
        const uint64_t row = c / kcp;
        const uint32_t ch = (uint32_t)(c - row * kcp);
        s16u32x4* out = reinterpret_cast<s16u32x4*>(body + c * kSplitChunkHalves);
        if (ch >= kc) {
#pragma unroll
            for (int q = 0; q < 3; ++q) out[q] = s16u32x4{0u, 0u, 0u, 0u};
            continue;
        }
        const f32x4* src = reinterpret_cast<const f32x4*>(x + row * k + 8ull * ch);
        const f32x4 a = src[0];
        const f32x4 b = src[1];
        const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
        uint32_t p[3][8];
#pragma unroll
        for (int t8 = 0; t8 < 8; ++t8) s16_split<DT>(v[t8], p[0][t8], p[1][t8], p[2][t8]);
#pragma unroll
        for (int q = 0; q < 3; ++q)
            out[q] = s16u32x4{p[q][0] | (p[q][1] << 16), p[q][2] | (p[q][3] << 16), p[q][4] | (p[q][5] << 16),
                              p[q][6] | (p[q][7] << 16)};
    }
}

template <int DT>
__global__ __launch_bounds__(256) void split_x_kernel(const float* __restrict__ x, uint32_t k, uint64_t rows,
                                                      uint16_t* __restrict__ xs) {
    split_x_chunks<DT>(x, k, rows, xs, (uint64_t)blockIdx.x * blockDim.x + threadIdx.x,
                       (uint64_t)gridDim.x * blockDim.x);
}

// The Grouped route's two preparations in one launch, side by side: blocks
// 0 .. n_experts build the id -> row map (the one-launch form, block e for
// key e), the blocks after them split the activations.  Neither reads what
// the other writes.
template <int DT>
__global__ __launch_bounds__(64 * kMapKeyedWaves) void map_split_x_kernel(
    const uint32_t* __restrict__ ids, uint32_t routed_rows, uint32_t n_experts, uint32_t span,
    uint32_t* __restrict__ counts, uint32_t* __restrict__ offsets, uint32_t* __restrict__ rows,
    const float* __restrict__ x, uint32_t k, uint64_t in_rows, uint16_t* __restrict__ xs) {
    const uint32_t map_blocks = n_experts + 1;
    if (blockIdx.x < map_blocks) {
        map_keyed_block(blockIdx.x, ids, routed_rows, n_experts, span, counts, offsets, rows);
        return;
    }
    split_x_chunks<DT>(x, k, in_rows, xs, (uint64_t)(blockIdx.x - map_blocks) * blockDim.x + threadIdx.x,
                       (uint64_t)(gridDim.x - map_blocks) * blockDim.x);
}

// A buffer offset past every extent: a buffer load there returns zeros.
constexpr uint32_t kOob = 0x80000000u;

__device__ __forceinline__ __amdgpu_buffer_rsrc_t s16_rsrc(const void* base, uint32_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}
__device__ __forceinline__ s16u32x4 s16_load(__amdgpu_buffer_rsrc_t r, uint32_t off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

// ---------------------------------------------------------------- Direct
// One wavefront per (routed row, 32 columns): the row is live in tile row 0
// (lanes 0, 16, 32, 48 supply its parts; the other lanes load zeros), two
// 16-column tiles.  Operands are loaded two rounds ahead, every round the
// same loads (past the last round, or past k, they return zeros).
constexpr int kDs16Cols = 32;

template <int DT>
__global__ __launch_bounds__(64) void direct_split16_kernel(MatmulArgs a, uint32_t xsplit_bytes) {
    const uint32_t n = a.n, k = a.k, kc = a.k / 8, kcp = s16_row_chunks(a.k);
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
    const bool live = l16 == 0;
    const __amdgpu_buffer_rsrc_t xrs = s16_rsrc(a.xsplit, xsplit_bytes);
    const uint32_t xbase = kZeroHalves * 2 + xr * kcp * 48 + (uint32_t)g * 48;  // this lane's chunk 0
    const __amdgpu_buffer_rsrc_t wrs =
        s16_rsrc(static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride, n * k * 2);
    uint32_t woff[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) woff[ct] = min(c0 + 16 * ct + l16, n - 1) * k * 2 + (uint32_t)g * 16;
    const uint32_t rounds = (k + 127) / 128;
    struct Ops {
        s16u32x4 x[kStepsPerRound][3];
        s16u32x4 w[kStepsPerRound][2];
    };
    auto load = [&](uint32_t q, Ops& o) {
        const bool inq = q < rounds;
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s) {
            const uint32_t step = 16 * q + 4 * s;  // first chunk of the step
            const uint32_t xo = live && inq ? xbase + step * 48 : kOob;
#pragma unroll
            for (int p = 0; p < 3; ++p) o.x[s][p] = s16_load(xrs, xo + 16 * p);
            const bool wk = inq && step + g < kc;
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) o.w[s][ct] = s16_load(wrs, wk ? woff[ct] + step * 16 : kOob);
        }
    };
    f32x4 hi[2], lo[2];
#pragma unroll
    for (int ct = 0; ct < 2; ++ct) hi[ct] = lo[ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    auto compute = [&](const Ops& o) {
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s)
#pragma unroll
            for (int ct = 0; ct < 2; ++ct) {
                hi[ct] = s16_mfma<DT>(o.x[s][0], o.w[s][ct], hi[ct]);
                lo[ct] = s16_mfma<DT>(o.x[s][1], o.w[s][ct], lo[ct]);
                lo[ct] = s16_mfma<DT>(o.x[s][2], o.w[s][ct], lo[ct]);
            }
    };
    // two register slots with static names, each refilled two rounds ahead
    Ops o0, o1;
    load(0, o0);
    load(1, o1);
    for (uint32_t q = 0; q < rounds; q += 2) {
        compute(o0);
        load(q + 2, o0);
        if (q + 1 < rounds) compute(o1);
        load(q + 3, o1);
    }
    // tile row 0: register 0 of lanes 0..15
    if (g == 0) {
#pragma unroll
        for (int ct = 0; ct < 2; ++ct) {
            const uint32_t col = c0 + 16 * ct + l16;
            if (col < n) yrow[col] = hi[ct][0] + lo[ct][0];
        }
    }
}

// ---------------------------------------------------------------- Grouped
// A job is 32 gathered rows of one expert (two 16-row tiles) by 64*CT
// output columns; a block of 4 wavefronts takes 16*CT columns each (CT
// 16-column tiles; more columns per job read the activation tile fewer
// times).  Per round of 128 k the block stages the split activations of its
// 32 rows in LDS; each wavefront's weights go straight into registers.  The
// rounds of all the jobs a block walks form one stream, its loads two rounds
// ahead.
constexpr int kGs16BM = 32;
constexpr int kGs16Waves = 4;
constexpr int kGs16Threads = 64 * kGs16Waves;
constexpr int kGs16RowBytes = 16 * 48 + 16;               // one row's 16 chunks of a round, padded
constexpr int kGs16Buf = kGs16BM * kGs16RowBytes;          // one round's activation tile
constexpr int kGs16Bufs = 3;
constexpr int kGs16Xcds = 8;

struct Gs16Job {
    uint32_t e, rc, col0, rbase;
};

template <int DT, int CT>
__global__ __launch_bounds__(kGs16Threads, 1) void grouped_split16_kernel(MatmulArgs a, uint32_t xsplit_bytes,
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
    const uint32_t n = a.n, k = a.k, kc = a.k / 8, kcp = s16_row_chunks(a.k);
    constexpr uint32_t BN = 64 * CT;
    const uint32_t ntiles = (n + BN - 1) / BN;
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
    auto decode = [&](uint32_t i) {  // block-uniform: the fields live in scalar registers
        const uint32_t jb = job0 + i * per_xcd;
        uint32_t e = 0;
        for (uint32_t st = top; st; st >>= 1)
            if (e + st < buckets && job_start[e + st] <= jb) e += st;
        e = __builtin_amdgcn_readfirstlane(e);
        const uint32_t local = jb - __builtin_amdgcn_readfirstlane(job_start[e]);
        const uint32_t mt = local / ntiles, nt = local - mt * ntiles;
        Gs16Job j;
        j.e = e;
        j.rc = min((uint32_t)kGs16BM, __builtin_amdgcn_readfirstlane(cnt_s[e]) - mt * kGs16BM);
        j.col0 = nt * BN;
        j.rbase = __builtin_amdgcn_readfirstlane(off_s[e]) + mt * kGs16BM;
        return j;
    };

    // ---- load side.  Staging: a round's activation tile is 32 rows x 48
    // pieces of 16 bytes (16 chunks x 3 parts, contiguous in the split
    // buffer and in LDS); thread t stages pieces t + 256 j (j < 6), so
    // consecutive lanes read consecutive pieces of a row.  Rows past the
    // job's rows read past the buffer (zeros).  Weights: this lane's columns.
    constexpr int kPieces = kGs16BM * 48 / kGs16Threads;  // 6 per thread
    const __amdgpu_buffer_rsrc_t xrs = s16_rsrc(a.xsplit, xsplit_bytes);
    uint32_t prow[kPieces], pm[kPieces], lds_piece[kPieces];
#pragma unroll
    for (int jj = 0; jj < kPieces; ++jj) {
        const uint32_t P = (uint32_t)tid + kGs16Threads * jj;
        prow[jj] = P / 48;
        pm[jj] = P - prow[jj] * 48;
        lds_piece[jj] = prow[jj] * kGs16RowBytes + pm[jj] * 16;
    }
    struct LoadJob {
        __amdgpu_buffer_rsrc_t w;    // the expert's matrix
        uint32_t xoff[kPieces];      // this thread's pieces in round 0 (past the buffer for empty rows)
        uint32_t woff[CT];           // this lane's weight columns, its chunk of a step
    };
    struct StageRows {
        uint32_t r[kPieces];
    };
    // the routed rows of this thread's pieces for job j (read one job ahead)
    auto stage_row = [&](const Gs16Job& j) {
        StageRows sr;
#pragma unroll
        for (int jj = 0; jj < kPieces; ++jj) sr.r[jj] = rows[j.rbase + (prow[jj] < j.rc ? prow[jj] : 0u)];
        return sr;
    };
    auto load_job = [&](const Gs16Job& j, const StageRows& sr) {
        LoadJob L;
#pragma unroll
        for (int jj = 0; jj < kPieces; ++jj) {
            const uint32_t xr = a.layout == 1 ? sr.r[jj] : sr.r[jj] / a.top_k;
            L.xoff[jj] = prow[jj] < j.rc ? kZeroHalves * 2 + xr * kcp * 48 + pm[jj] * 16 : kOob;
        }
        const uint32_t wexp = j.e < a.n_experts ? j.e : 0u;
        L.w = s16_rsrc(static_cast<const uint8_t*>(a.weights) + (size_t)wexp * a.stride, n * k * 2);
#pragma unroll
        for (int ct = 0; ct < CT; ++ct)
            L.woff[ct] = min(j.col0 + 16 * CT * wave + 16 * ct + l16, n - 1) * k * 2 + (uint32_t)g * 16;
        return L;
    };
    struct Stage {
        s16u32x4 x[kPieces];    // this thread's staged pieces
        s16u32x4 w[kStepsPerRound][CT];
    };
    // Every position issues the same loads; past k, and past the end of the
    // stream, they read at an offset past the buffer and return zeros (the
    // activation rows are also padded with zero chunks).  With the same
    // number of loads in flight on every path, each wait before the
    // matrix-core steps covers exactly the loads it needs.
    auto load_round = [&](const LoadJob& L, uint32_t q, bool live, Stage& st) {
#pragma unroll
        for (int jj = 0; jj < kPieces; ++jj) st.x[jj] = s16_load(xrs, live ? L.xoff[jj] + q * 16 * 48 : kOob);
#pragma unroll
        for (int s = 0; s < kStepsPerRound; ++s) {
            const uint32_t step = 16 * q + 4 * s;
            const bool wk = live && step + g < kc;
#pragma unroll
            for (int ct = 0; ct < CT; ++ct) st.w[s][ct] = s16_load(L.w, wk ? L.woff[ct] + step * 16 : kOob);
        }
    };
    auto store_x = [&](int buf, const Stage& st) {
        uint8_t* dst = xbuf + buf * kGs16Buf;
#pragma unroll
        for (int jj = 0; jj < kPieces; ++jj) *reinterpret_cast<s16u32x4*>(dst + lds_piece[jj]) = st.x[jj];
    };

    // ---- compute side: per output tile a hi chain (first parts) and a lo
    // chain (second then third parts), both from +0 over the whole job
    f32x4 hi[2][CT], lo[2][CT];
    auto compute_round = [&](int buf, const Stage& st) {
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
                for (int ct = 0; ct < CT; ++ct) {
                    hi[rt][ct] = s16_mfma<DT>(xa[rt][0], st.w[s][ct], hi[rt][ct]);
                    lo[rt][ct] = s16_mfma<DT>(xa[rt][1], st.w[s][ct], lo[rt][ct]);
                    lo[rt][ct] = s16_mfma<DT>(xa[rt][2], st.w[s][ct], lo[rt][ct]);
                }
        }
    };
    // The output rows of this lane's results, read when the job starts.
    // The job's 32 row-list entries are read with block-uniform (scalar)
    // loads, whose wait does not hold up the vector loads in flight; the
    // row list has 32 spare entries past its end, so the read stays in
    // bounds for the last bucket (entries past the job's rows are not used).
    uint32_t yrows[2][4];
    auto read_yrows = [&](const Gs16Job& j) {
        uint32_t ent[kGs16BM];
#pragma unroll
        for (int i = 0; i < kGs16BM; ++i) ent[i] = __builtin_amdgcn_readfirstlane(rows[j.rbase + i]);
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int i = 16 * rt + v;
                yrows[rt][v] = g == 0 ? ent[i] : g == 1 ? ent[i + 4] : g == 2 ? ent[i + 8] : ent[i + 12];
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
                for (int ct = 0; ct < CT; ++ct) {
                    const uint32_t col = j.col0 + 16 * CT * wave + 16 * ct + l16;
                    if (col < n) yrow[col] = nan_rows ? quiet_nan() : hi[rt][ct][v] + lo[rt][ct][v];
                }
            }
    };

    // The stream: position i = (job i / R, round i % R).  Position i is
    // computed from LDS buffer i % 3 and register slot i % 3; its loads were
    // issued at position i - 2 and its activations stored to LDS at
    // position i - 1 (before that position's barrier).
    const uint32_t total_pos = my_jobs * R;
    Gs16Job jc = decode(0);             // job being computed
    read_yrows(jc);
    LoadJob Lj = load_job(jc, stage_row(jc));  // job being loaded
    uint32_t lj = 0, lq = 0;            // its job index and round
    StageRows next_rr = stage_row(decode(my_jobs > 1 ? 1u : 0u));  // staged rows of job lj + 1
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
    load_round(Lj, lq, true, ring0);
    advance_load();
    load_round(Lj, lq, total_pos > 1, ring1);
    if (total_pos > 1) advance_load();
    store_x(0, ring0);
    __syncthreads();
#pragma unroll
    for (int rt = 0; rt < 2; ++rt)
#pragma unroll
        for (int ct = 0; ct < CT; ++ct) hi[rt][ct] = lo[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    uint32_t q = 0;  // round of the computed job
    uint32_t ci = 0;
    // Position i: load position i + 2 into slot (i + 2) % 3; compute from
    // LDS buffer and register slot i % 3; store position i + 1's staged
    // activations into LDS buffer (i + 1) % 3; one barrier.
    auto position = [&](uint32_t i, int buf, Stage& cur, Stage& nxt, Stage& ahead) __attribute__((always_inline)) {
        const bool live = i + 2 < total_pos;
        load_round(Lj, lq, live, ahead);
        if (live) advance_load();
        compute_round(buf, cur);
        if (i + 1 < total_pos) store_x(buf == 2 ? 0 : buf + 1, nxt);
        if (++q == R) {
            finish(jc);
#pragma unroll
            for (int rt = 0; rt < 2; ++rt)
#pragma unroll
                for (int ct = 0; ct < CT; ++ct) hi[rt][ct] = lo[rt][ct] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
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

uint64_t split16_bytes(uint64_t in_rows, uint32_t k) {
    return (uint64_t)kZeroHalves * 2 + in_rows * s16_row_chunks(k) * kSplitChunkHalves * 2;
}

bool map_split16_x_fits(const MatmulArgs& a) { return map_keyed_fits(a.m * a.top_k, a.n_experts); }

hipError_t launch_map_split16_x(const MatmulArgs& a, const MapBuffers& buf, hipStream_t stream) {
    const uint32_t routed = a.m * a.top_k;
    const uint64_t in_rows = a.layout == 1 ? (uint64_t)routed : a.m;
    const uint64_t chunks = in_rows * s16_row_chunks(a.k);
    constexpr uint32_t threads = 64 * kMapKeyedWaves;
    uint64_t split_blocks = (chunks + threads - 1) / threads;
    if (split_blocks > 4096) split_blocks = 4096;
    if (split_blocks == 0) split_blocks = 1;
    const uint32_t grid = a.n_experts + 1 + (uint32_t)split_blocks;
    const uint32_t span = map_keyed_span(routed);
    if (a.dtype == kDtypeF16)
        hipLaunchKernelGGL(map_split_x_kernel<kDtypeF16>, dim3(grid), dim3(threads), 0, stream, a.ids, routed,
                           a.n_experts, span, buf.counts, buf.offsets, buf.rows, a.input, a.k, in_rows, a.xsplit);
    else
        hipLaunchKernelGGL(map_split_x_kernel<kDtypeBF16>, dim3(grid), dim3(threads), 0, stream, a.ids, routed,
                           a.n_experts, span, buf.counts, buf.offsets, buf.rows, a.input, a.k, in_rows, a.xsplit);
    return launched(EIDM_KERNEL_MAP_SPLIT_X, grid, threads, 0);
}

hipError_t launch_split16_x(const MatmulArgs& a, hipStream_t stream) {
    const uint64_t in_rows = a.layout == 1 ? (uint64_t)a.m * a.top_k : a.m;
    const uint64_t chunks = in_rows * s16_row_chunks(a.k);
    uint64_t blocks = (chunks + 255) / 256;
    if (blocks > 16384) blocks = 16384;
    if (blocks == 0) blocks = 1;
    if (a.dtype == kDtypeF16)
        hipLaunchKernelGGL(split_x_kernel<kDtypeF16>, dim3((uint32_t)blocks), dim3(256), 0, stream, a.input, a.k,
                           in_rows, a.xsplit);
    else
        hipLaunchKernelGGL(split_x_kernel<kDtypeBF16>, dim3((uint32_t)blocks), dim3(256), 0, stream, a.input, a.k,
                           in_rows, a.xsplit);
    return launched(EIDM_KERNEL_SPLIT_X, (uint32_t)blocks, 256, 0);
}

// buffer loads take 32-bit offsets: each expert's matrix and the split
// activations must span less than 2 GiB (checked when the shape is
// validated)
static uint32_t split_bytes_of(const MatmulArgs& a) {
    const uint64_t in_rows = a.layout == 1 ? (uint64_t)a.m * a.top_k : a.m;
    return (uint32_t)split16_bytes(in_rows, a.k);
}

hipError_t launch_direct_split16(const MatmulArgs& a, hipStream_t stream) {
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t blocks = routed * ((a.n + kDs16Cols - 1) / kDs16Cols);
    if (blocks > 0x7fffffffull) return hipErrorInvalidValue;
    const uint32_t xb = split_bytes_of(a);
    if (a.dtype == kDtypeF16)
        hipLaunchKernelGGL(direct_split16_kernel<kDtypeF16>, dim3((uint32_t)blocks), dim3(64), 0, stream, a, xb);
    else
        hipLaunchKernelGGL(direct_split16_kernel<kDtypeBF16>, dim3((uint32_t)blocks), dim3(64), 0, stream, a, xb);
    return launched(EIDM_KERNEL_DIRECT_SPLIT16, (uint32_t)blocks, 64, 0);
}

template <int DT, int CT>
hipError_t launch_gs16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream) {
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t ntiles = (a.n + 64 * CT - 1) / (64 * CT);
    const uint64_t job_bound = (routed / kGs16BM + a.n_experts + 1) * ntiles;
    const size_t lds = (size_t)kGs16Bufs * kGs16Buf + (3 * (size_t)a.n_experts + 4) * sizeof(uint32_t);
    auto kernel = grouped_split16_kernel<DT, CT>;
    static std::atomic<bool> raised{false};
    if (!raised.load(std::memory_order_relaxed)) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        raised.store(true, std::memory_order_relaxed);
    }
    const uint64_t resident = (uint64_t)(device_cus > 0 ? device_cus : 256);
    uint64_t grid = job_bound < resident ? job_bound : resident;
    grid = (grid + kGs16Xcds - 1) / kGs16Xcds * kGs16Xcds;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kGs16Threads), lds, stream, a, split_bytes_of(a), buf.counts,
                       buf.offsets, buf.rows);
    return launched(EIDM_KERNEL_GROUPED_SPLIT16, (uint32_t)grid, kGs16Threads, (uint32_t)lds);
}

// Columns per wavefront: 3 16-column tiles when that job count (estimated
// from the routed rows, as whole 32-row tiles) gives the busiest compute
// unit no more work than 2 tiles would, else 2.  (4 tiles spill registers
// and measured slower.)
int gs16_column_tiles(const MatmulArgs& a, int device_cus) {
    const uint64_t row_tiles = ((uint64_t)a.m * a.top_k + kGs16BM - 1) / kGs16BM;
    const uint64_t cus = (uint64_t)(device_cus > 0 ? device_cus : 256);
    auto makespan = [&](uint64_t ct) {
        const uint64_t jobs = row_tiles * ((a.n + 64 * ct - 1) / (64 * ct));
        return (jobs + cus - 1) / cus * ct;  // jobs of the busiest unit x columns per job
    };
    return makespan(3) <= makespan(2) ? 3 : 2;
}

hipError_t launch_grouped_split16(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream) {
    const int ct = gs16_column_tiles(a, device_cus);
    if (a.dtype == kDtypeF16)
        return ct == 3 ? launch_gs16<kDtypeF16, 3>(a, buf, device_cus, stream)
                       : launch_gs16<kDtypeF16, 2>(a, buf, device_cus, stream);
    return ct == 3 ? launch_gs16<kDtypeBF16, 3>(a, buf, device_cus, stream)
                   : launch_gs16<kDtypeBF16, 2>(a, buf, device_cus, stream);
}

}  // namespace eidm
