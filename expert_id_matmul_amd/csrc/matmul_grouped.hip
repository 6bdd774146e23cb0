// matmul_grouped.hip -- Grouped form of the expert-ID matmul: the routed rows
// of each expert (from the id -> row map) are gathered into tiles of BM rows
// x BN columns, and each tile is one job of a persistent grid.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: fn expected_dispatches
// gives the grouped route a map dispatch and then tiles of (rows of one
// expert) x (output columns); the value-independence theorem statement
// requires it to produce the Direct route's bits, differing only in which
// independent rows are computed together.
//
// Every output goes through the same canonical order as in the Direct form
// (eidm_device.hpp): the 16 blocks of each matrix-core step are the 16
// k-slices; within a block the 4 A-rows are 4 gathered routed rows and the 4
// B-columns are 4 output columns.  So one step advances 16 outputs of every
// slice at once, and one wavefront holding a (4R rows) x (4C columns) tile
// issues R*C steps per k element of its slices.
//
// Block = WAVES wavefronts side by side along n: tile BM = 4R rows by
// BN = 4C*WAVES columns.  Per round (128 k):
//   * the gathered activation tile [BM][128] f32 goes through LDS, double
//     buffered (the next round is loaded into registers while this one is
//     computed, then written to the other buffer); 16-byte chunks are
//     XOR-swizzled by row so the per-lane reads spread over the banks;
//   * each wavefront reads its own weight columns straight from global memory
//     into a two-round register ring (no reuse across wavefronts, so no LDS).
// The 16 slice sums of each output are combined by a recursive-halving
// exchange that keeps the canonical pairing (b with b^8, then b^4, b^2,
// b^1) and leaves each lane with R*C/4 finished outputs.
//
// Jobs are numbered expert-major (bucket e, row tile mt, column tile nt),
// column tile fastest; the block ids are remapped so that the blocks
// resident on one XCD (the hardware deals blocks to the 8 XCDs round-robin)
// walk a contiguous range of jobs and share that expert's weights (and a row
// tile's activations) in their L2.  Each block reads the map's per-expert counts and scans them itself.
// The last bucket (ids >= n_experts) gets quiet NaN rows.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

#ifndef EIDM_GROUPED_R
#define EIDM_GROUPED_R 4
#endif
#ifndef EIDM_GROUPED_C
#define EIDM_GROUPED_C 4
#endif
#ifndef EIDM_GROUPED_WAVES
#define EIDM_GROUPED_WAVES 8
#endif

namespace eidm {
namespace {

constexpr int kXcds = 8;

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

template <int DT> struct Pieces { static constexpr int value = DtypeSize<DT>::value / 2; };

template <int V> struct IntC { static constexpr int value = V; };
static_assert(EIDM_GROUPED_R == 4 || EIDM_GROUPED_R == 8, "row-group dispatch covers R = 4 and R = 8");

// 16-byte chunk swizzle of the activation tile: row r's chunk c is stored at
// chunk c ^ {0, 1, 8, 9}[r & 3] (rows are 32 chunks = 512 bytes), so the 16
// lanes (4 slices x 4 rows) of one read touch 16 different chunk columns.
__device__ __forceinline__ int swz(int row, int chunk) {
    const int t = row & 3;
    return chunk ^ ((t & 1) | ((t & 2) << 2));  // 0, 1, 8, 9
}

template <int DT>
__device__ __forceinline__ void load_w_pieces(const uint8_t* row, int kk, u32x4 (&p)[Pieces<DT>::value]) {
    constexpr int S = DtypeSize<DT>::value;
#pragma unroll
    for (int i = 0; i < Pieces<DT>::value; ++i)
        p[i] = *(reinterpret_cast<const u32x4*>(row + (size_t)kk * S) + i);
}

// The slice sums' recursive halving over lane bits 5, 4, 3, 2 (slices b with
// b^8, then b^4, b^2, b^1): at each level a lane keeps half of its values and
// adds its partner's copy of that half, so afterwards lane (b, q) holds
// values NV/16*b .. NV/16*b + NV/16 - 1.  Lane bits 5 and 4 use the gfx950
// half-wave and row swaps (one swap gives each lane its partner's half),
// bits 3 and 2 DPP row rotations and shifts; the sums are those of the
// cross-lane shuffle form (f32 addition is commutative).
// f32 value of lane (DPP control CTRL) of this row; lanes whose source lies
// outside the row read 0 (their results are never kept).
template <int CTRL>
__device__ __forceinline__ float dpp_f32(float v) {
    return __int_as_float(__builtin_amdgcn_mov_dpp(__float_as_int(v), CTRL, 0xf, 0xf, true));
}

template <int NV>
__device__ __forceinline__ void halving_exchange(float (&val)[NV], int lane) {
    {
        constexpr int half = NV / 2;  // lane bit 5: halves of the wave
#pragma unroll
        for (int jj = 0; jj < half; ++jj) {
            const auto r = __builtin_amdgcn_permlane32_swap(__float_as_uint(val[jj]), __float_as_uint(val[half + jj]),
                                                            false, false);
            val[jj] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    }
    {
        constexpr int half = NV / 4;  // lane bit 4: rows of 16
#pragma unroll
        for (int jj = 0; jj < half; ++jj) {
            const auto r = __builtin_amdgcn_permlane16_swap(__float_as_uint(val[jj]), __float_as_uint(val[half + jj]),
                                                            false, false);
            val[jj] = __uint_as_float(r[0]) + __uint_as_float(r[1]);
        }
    }
    {
        // lane bit 3: the partner is 8 lanes away in the same row, which a
        // row rotation by 8 reaches from every lane; each half of the row
        // adds the partner's copy of the value it keeps (the other half's
        // sum is discarded)
        constexpr int half = NV / 8;
        const bool upper = (lane & 8) != 0;
#pragma unroll
        for (int jj = 0; jj < half; ++jj) {
            const float lo = val[jj] + dpp_f32<0x128>(val[jj]);                   // row_ror:8
            const float hi = val[half + jj] + dpp_f32<0x128>(val[half + jj]);
            val[jj] = upper ? hi : lo;
        }
    }
    {
        // lane bit 2: lanes 4 apart within each 8, reached by a row shift
        // left (lower lanes) or right (upper lanes) by 4
        constexpr int half = NV / 16;
        const bool upper = (lane & 4) != 0;
#pragma unroll
        for (int jj = 0; jj < half; ++jj) {
            const float lo = val[jj] + dpp_f32<0x104>(val[jj]);                   // row_shl:4
            const float hi = val[half + jj] + dpp_f32<0x114>(val[half + jj]);     // row_shr:4
            val[jj] = upper ? hi : lo;
        }
    }
}

template <int DT>
__device__ __forceinline__ void widen_w_pieces(const u32x4 (&p)[Pieces<DT>::value], float (&w)[kGranule]) {
    if constexpr (DT == kDtypeF32) {
        w[0] = __uint_as_float(p[0].x); w[1] = __uint_as_float(p[0].y);
        w[2] = __uint_as_float(p[0].z); w[3] = __uint_as_float(p[0].w);
        w[4] = __uint_as_float(p[1].x); w[5] = __uint_as_float(p[1].y);
        w[6] = __uint_as_float(p[1].z); w[7] = __uint_as_float(p[1].w);
    } else {
        widen_pair<DT>(p[0].x, w[0], w[1]);
        widen_pair<DT>(p[0].y, w[2], w[3]);
        widen_pair<DT>(p[0].z, w[4], w[5]);
        widen_pair<DT>(p[0].w, w[6], w[7]);
    }
}

// One round's weight granules for this lane's C columns (whole 16-byte
// granules of a vector round).
template <int DT, int C>
struct WeightRound {
    u32x4 p[C][Pieces<DT>::value];
};

// This thread's share of one round's activation tile.
template <int N>
struct XTile {
    f32x4 v[N];
};

template <int DT, int C>
__device__ __forceinline__ void widen_w_pieces_all(const WeightRound<DT, C>& wr, float (&w)[C][kGranule]) {
#pragma unroll
    for (int c = 0; c < C; ++c) widen_w_pieces<DT>(wr.p[c], w[c]);
}

template <int DT, int R, int C, int WAVES>
__global__ __launch_bounds__(64 * WAVES) void grouped_kernel(MatmulArgs a,
                                                                const uint32_t* __restrict__ counts,
                                                                const uint32_t* __restrict__ offsets,
                                                                const uint32_t* __restrict__ rows) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int BM = 4 * R, BN = 4 * C * WAVES;
    constexpr int XCHUNKS = BM * (kRoundK / 4);          // 16-byte chunks per activation tile
    static_assert(XCHUNKS % THREADS == 0, "activation tile must split evenly");
    constexpr int XPER = XCHUNKS / THREADS;              // chunks per thread per round

    extern __shared__ __align__(16) uint8_t smem[];
    float* xs = reinterpret_cast<float*>(smem);          // [2][BM][128]
    uint32_t* job_start = reinterpret_cast<uint32_t*>(smem + 2 * BM * kRoundK * sizeof(float));
    __shared__ uint32_t wave_tot[WAVES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = lane >> 2, q = lane & 3;
    const uint32_t buckets = a.n_experts + 1;
    const uint32_t ntiles = (a.n + BN - 1) / BN;
    const int n = (int)a.n, k = (int)a.k;

    // jobs per bucket -> exclusive prefix in LDS
    {
        const uint32_t per = (buckets + THREADS - 1) / THREADS;
        const uint32_t begin = min(buckets, (uint32_t)tid * per);
        const uint32_t end = min(buckets, begin + per);
        uint32_t s = 0;
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t jobs = ((counts[i] + BM - 1) / BM) * ntiles;
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
        for (int w = 0; w < WAVES; ++w) {
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
    const int rounds = (k + kRoundK - 1) / kRoundK;
    const int full = a.vec ? k / kRoundK : 0;  // vector rounds (whole aligned granules)
    // XCD-contiguous job walk (the grid is a multiple of 8 blocks)
    const uint32_t per_xcd = gridDim.x / kXcds;
    const uint32_t vblock = (blockIdx.x % kXcds) * per_xcd + blockIdx.x / kXcds;

    for (uint32_t job = vblock; job < total_jobs; job += gridDim.x) {
        uint32_t lo = 0, hi = buckets;  // job_start[lo] <= job < job_start[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (job_start[mid] <= job) lo = mid; else hi = mid;
        }
        const uint32_t e = lo;
        const uint32_t local = job - job_start[e];
        const uint32_t mt = local / ntiles, nt = local % ntiles;
        const uint32_t row_begin = offsets[e] + mt * BM;
        const int row_count = (int)min((uint32_t)BM, counts[e] - mt * BM);
        const int col_base = (int)(nt * BN) + wave * 4 * C;

        if (e == a.n_experts) {  // ids naming no expert: NaN rows
            for (int i = tid; i < BM * BN; i += THREADS) {
                const int lr = i / BN, col = (int)(nt * BN) + i % BN;
                if (lr < row_count && col < n)
                    a.output[(size_t)rows[row_begin + lr] * a.n + col] = quiet_nan();
            }
            continue;
        }

        // ---- activation staging: this thread's XPER chunks (rows tid/32 + j*THREADS/32)
        const float* xsrc[XPER];
        bool xvalid[XPER];
        int xrow_l[XPER], xchunk[XPER];
        // rows past row_count read the tile's first row: their outputs are
        // never stored, and the loads stay branch-free
#pragma unroll
        for (int j = 0; j < XPER; ++j) {
            const int id = tid + j * THREADS;
            xrow_l[j] = id >> 5;
            xchunk[j] = id & 31;
            xvalid[j] = xrow_l[j] < row_count;
            const uint32_t rho = rows[row_begin + (xvalid[j] ? xrow_l[j] : 0)];
            const uint32_t xr = a.layout == 1 ? rho : rho / a.top_k;
            xsrc[j] = a.input + (size_t)xr * a.k + xchunk[j] * 4;
        }
        // whole 16-byte chunks of a vector round (every lane, no masks)
        auto load_x_vec = [&](int g) {
            XTile<XPER> t;
#pragma unroll
            for (int j = 0; j < XPER; ++j) t.v[j] = *reinterpret_cast<const f32x4*>(xsrc[j] + g * kRoundK);
            return t;
        };
        // masked chunks: zero past k (the k tail) and for rows past row_count
        auto load_x_masked = [&](int g) {
            XTile<XPER> t;
#pragma unroll
            for (int j = 0; j < XPER; ++j) {
                const int kk = g * kRoundK + xchunk[j] * 4;
                const float* p = xsrc[j] + g * kRoundK;
#pragma unroll
                for (int i = 0; i < 4; ++i) t.v[j][i] = xvalid[j] && kk + i < k ? p[i] : 0.0f;
            }
            return t;
        };
        auto load_x = [&](int g) { return g < full ? load_x_vec(g) : load_x_masked(g); };
        auto store_x = [&](int buf, const XTile<XPER>& t) {
#pragma unroll
            for (int j = 0; j < XPER; ++j) {
                float* dst = xs + ((size_t)buf * BM + xrow_l[j]) * kRoundK + swz(xrow_l[j], xchunk[j]) * 4;
                *reinterpret_cast<f32x4*>(dst) = t.v[j];
            }
        };

        // ---- this lane's weight columns
        const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;
        const uint8_t* wrow[C];
        bool cvalid[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int col = col_base + 4 * c + q;
            cvalid[c] = col < n;
            wrow[c] = wexp + (size_t)(cvalid[c] ? col : 0) * a.k * DtypeSize<DT>::value;
        }
        auto fetch_w_vec = [&](int g, WeightRound<DT, C>& wr) {
#pragma unroll
            for (int c = 0; c < C; ++c) load_w_pieces<DT>(wrow[c], g * kRoundK + b * kGranule, wr.p[c]);
        };
        auto fetch_w = [&](int g, WeightRound<DT, C>& wr) {
            if (g < full) fetch_w_vec(g, wr);
        };
        auto widen_w = [&](int g, const WeightRound<DT, C>& wr, float (&w)[C][kGranule]) {
            if (g < full) {
#pragma unroll
                for (int c = 0; c < C; ++c) widen_w_pieces<DT>(wr.p[c], w[c]);
            } else {
#pragma unroll
                for (int c = 0; c < C; ++c)
                    load_weight_granule<DT>(wrow[c], g * kRoundK + b * kGranule, k, cvalid[c], a.vec, w[c]);
            }
        };

        f32x4 acc[R][C];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        // one round from LDS buffer `buf`: k elements in pairs (8-byte reads),
        // each pair feeding R*C accumulation steps per element
        auto compute = [&](int buf, const float (&w)[C][kGranule]) {
            const float* xb = xs + (size_t)buf * BM * kRoundK;
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
                float2 xa[R];
#pragma unroll
                for (int r = 0; r < R; ++r) {
                    const int row = 4 * r + q;
                    const int chunk = swz(row, 2 * b + (pr >> 1));
                    xa[r] = *reinterpret_cast<const float2*>(xb + row * kRoundK + chunk * 4 + (pr & 1) * 2);
                }
#pragma unroll
                for (int i = 0; i < 2; ++i)
#pragma unroll
                    for (int r = 0; r < R; ++r) {
                        const float xv = i == 0 ? xa[r].x : xa[r].y;
#pragma unroll
                        for (int c = 0; c < C; ++c)
                            acc[r][c] = mfma_step(xv, w[c][2 * pr + i], acc[r][c]);
                    }
            }
        };

        // ---- software pipeline over rounds.  Load order per round: the
        // next round's activations, then the weights two rounds ahead, so the
        // wait for the activations (before their LDS store) never waits for
        // the younger weight loads.
        WeightRound<DT, C> ring[2];
        {
            const XTile<XPER> t = load_x(0);
            fetch_w(0, ring[0]);
            fetch_w(1, ring[1]);
            __syncthreads();  // the previous job is done with both buffers
            store_x(0, t);
        }
        __syncthreads();
        int g = 0;
        // steady state: vector rounds with both refills, no branches
        for (; g + 4 <= full; g += 2) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int gg = g + d;
                const XTile<XPER> t = load_x_vec(gg + 1);
                __builtin_amdgcn_sched_barrier(0);
                float w[C][kGranule];
                widen_w_pieces_all<DT, C>(ring[d], w);
                __builtin_amdgcn_sched_barrier(0);
                fetch_w_vec(gg + 2, ring[d]);
                __builtin_amdgcn_sched_barrier(0);
                compute(d, w);
                __builtin_amdgcn_sched_barrier(0);
                store_x(d ^ 1, t);
                __syncthreads();
            }
        }
        // the remaining rounds (k tail, unaligned rows, short k)
        for (; g < rounds; g += 2) {
#pragma unroll
            for (int d = 0; d < 2; ++d) {
                const int gg = g + d;
                if (gg < rounds) {
                    const bool more = gg + 1 < rounds;
                    XTile<XPER> t{};
                    if (more) t = load_x(gg + 1);
                    float w[C][kGranule];
                    widen_w(gg, ring[d], w);
                    fetch_w(gg + 2, ring[d]);
                    compute(d, w);
                    if (more) store_x(d ^ 1, t);
                    __syncthreads();
                }
            }
        }

        // ---- slice sums: recursive halving over lane bits 5, 4, 3, 2
        // value index o = (r*C + c)*4 + v; after the exchange lane (b, q)
        // holds o = PER*b + j, j < PER.
        constexpr int NV = R * C * 4;
        constexpr int PER = NV / 16;
        static_assert(NV % 16 == 0, "the exchange halves the values four times");
        float val[NV];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int v = 0; v < 4; ++v) val[(r * C + c) * 4 + v] = acc[r][c][v];
        halving_exchange<NV>(val, lane);
#pragma unroll
        for (int j = 0; j < PER; ++j) {
            const int o = PER * b + j;
            const int r = o / (4 * C), c = (o / 4) % C, v = o % 4;
            const int lr = 4 * r + v;
            const int col = col_base + 4 * c + q;
            if (lr < row_count && col < n)
                a.output[(size_t)rows[row_begin + lr] * a.n + col] = val[j];
        }
    }
}

// Streamed form, for vector rows (16-byte aligned, k a multiple of 4) of at
// least two rounds (at least three when their number is odd): the rounds of
// all the jobs one block walks are a single stream.  The loads of a job's
// first rounds are issued while the previous job computes its last ones; the
// job table (bucket counts, offsets, first job), the decoded job descriptors
// and the jobs' row-map entries are in LDS or registers, so a block never
// waits on a global read between jobs.  Arithmetic and order are those of
// grouped_kernel.  ODD: the number of
// rounds is odd (see run_job).  TAIL: k is not a multiple of 128, so the last
// round is partly past k.  Every 16-byte weight piece and 4-element
// activation chunk lies wholly before or past k (rows are whole 16-byte
// pieces); those past k enter as +0, as the documented order has it.  They
// are loaded from the same place one round earlier (in bounds, no branch
// around the load) and replaced by zeros where they are used: activations
// when stored to LDS, weights in the step that computes the job's last
// round (known at each call site).
template <int DT, int R, int C, int WAVES, bool ODD, bool TAIL>
__global__ __launch_bounds__(64 * WAVES) void grouped_stream_kernel(MatmulArgs a,
                                                                       const uint32_t* __restrict__ counts,
                                                                       const uint32_t* __restrict__ offsets,
                                                                       const uint32_t* __restrict__ rows) {
    constexpr int THREADS = 64 * WAVES;
    constexpr int BM = 4 * R, BN = 4 * C * WAVES;
    constexpr int XCHUNKS = BM * (kRoundK / 4);
    static_assert(XCHUNKS % THREADS == 0, "activation tile must split evenly");
    constexpr int XPER = XCHUNKS / THREADS;
    constexpr int S = DtypeSize<DT>::value;
    constexpr int NV = R * C * 4;
    constexpr int PER = NV / 16;
    static_assert(NV % 16 == 0, "the exchange halves the values four times");

    const uint32_t buckets = a.n_experts + 1;
    extern __shared__ __align__(16) uint8_t smem[];
    float* xs = reinterpret_cast<float*>(smem);          // [2 buffers][2 rounds][BM][128]
    uint32_t* job_start = reinterpret_cast<uint32_t*>(smem + 4 * BM * kRoundK * sizeof(float));
    uint32_t* cnt_s = job_start + buckets + 1;            // [buckets]
    uint32_t* off_s = cnt_s + buckets;                    // [buckets]
    uint32_t* rows_s = off_s + buckets;                   // [64 jobs][BM] row-map entries
    __shared__ uint32_t wave_tot[WAVES];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = lane >> 2, q = lane & 3;
    const uint32_t ntiles = (a.n + BN - 1) / BN;
    const int n = (int)a.n, k = (int)a.k;
    const int rounds = TAIL ? (k + kRoundK - 1) / kRoundK : k / kRoundK;
    const int last = rounds - 1;
    const int tail = k - last * kRoundK;  // elements of the last round inside k (TAIL)

    // job table: jobs per bucket -> exclusive prefix, with counts and offsets
    {
        const uint32_t per = (buckets + THREADS - 1) / THREADS;
        const uint32_t begin = min(buckets, (uint32_t)tid * per);
        const uint32_t end = min(buckets, begin + per);
        uint32_t s = 0;
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t c = counts[i];
            cnt_s[i] = c;
            off_s[i] = offsets[i];
            const uint32_t jobs = ((c + BM - 1) / BM) * ntiles;
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
        for (int w = 0; w < WAVES; ++w) {
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
    // Each XCD walks one contiguous eighth of the job list with its blocks
    // side by side (block l of the XCD takes jobs first + l + i*per_xcd), so
    // all row tiles of one (expert, column tile) meet in one L2 and the
    // weight columns are fetched from HBM once.
    const uint32_t per_xcd = gridDim.x / kXcds;             // blocks on one XCD
    const uint32_t xcd_jobs = (total_jobs + kXcds - 1) / kXcds;
    const uint32_t xcd = blockIdx.x % kXcds;
    const uint32_t job = xcd * xcd_jobs + blockIdx.x / kXcds;  // this block's first job
    const uint32_t job_end = min(total_jobs, (xcd + 1) * xcd_jobs);
    if (job >= job_end) return;  // the whole block leaves together

    struct Job {
        uint32_t e;          // bucket (n_experts = ids naming no expert)
        uint32_t wexp;       // expert whose weights are read (e, or 0 for that bucket)
        uint32_t col0;       // first output column of the tile
        uint32_t slot;       // its place in the decoded chunk (row-map entries in LDS)
        int row_count;
    };
    // Job descriptors.  The block's jobs are job + i*per_xcd < job_end.
    // A wavefront decodes 64 of them at once, one per lane, and keeps them in
    // three registers; a job is then three lane reads, so the per-job path
    // has no dependent chain of LDS lookups.  Lane L of a chunk starting at
    // index i0 holds job i0 + L: the bucket of job jb is the last e with
    // job_start[e] <= jb (job_start is non-decreasing; an empty bucket's start
    // equals the next one's), found by a fixed-length binary search.
    uint32_t top = 1;
    while (top * 2 <= buckets) top *= 2;  // largest power of two <= buckets
    uint32_t chunk_base = 0x80000000u;    // index of the job in lane 0 (none yet)
    uint32_t d_erc = 0, d_col0 = 0, d_rb = 0;  // bucket | row_count << 16, first column, first map entry
    // The chunk's row-map entries are copied into LDS in the same pass (the
    // block's threads share the 64 x BM loads), so a job's row indices are
    // LDS reads: no global read sits in the in-order load queue between two
    // jobs, where every later wait would wait for it too.
    constexpr int ENT = 64 * BM, EPT = (ENT + THREADS - 1) / THREADS;
    auto refill = [&](uint32_t i0) {
        chunk_base = i0;
        d_erc = 0;
        d_col0 = 0;
        d_rb = 0;
        const uint64_t jb64 = (uint64_t)job + ((uint64_t)i0 + (uint64_t)lane) * per_xcd;
        if (jb64 < job_end) {
            const uint32_t jb = (uint32_t)jb64;
            uint32_t e = 0;
            for (uint32_t st = top; st; st >>= 1)
                if (e + st < buckets && job_start[e + st] <= jb) e += st;
            const uint32_t cnt = cnt_s[e];
            const uint32_t local = jb - job_start[e];
            const uint32_t mt = local / ntiles, nt = local - mt * ntiles;
            d_erc = e | (min((uint32_t)BM, cnt - mt * BM) << 16);
            d_col0 = nt * BN;
            d_rb = off_s[e] + mt * BM;
        }
        // entry (L, lr): map entry lr of chunk job L (rows past its row count
        // read its first row); every wavefront decoded the same chunk
        uint32_t v[EPT];
#pragma unroll
        for (int jj = 0; jj < EPT; ++jj) {
            const int ent = tid + jj * THREADS;
            if (ent < ENT) {
                const int L = ent / BM, lr = ent % BM;
                const uint32_t rb = (uint32_t)__shfl((int)d_rb, L);
                const uint32_t rc = (uint32_t)__shfl((int)d_erc, L) >> 16;
                v[jj] = rows[rb + ((uint32_t)lr < rc ? (uint32_t)lr : 0u)];
            }
        }
#pragma unroll
        for (int jj = 0; jj < EPT; ++jj) {
            const int ent = tid + jj * THREADS;
            if (ent < ENT) rows_s[ent] = v[jj];
        }
        __syncthreads();
    };
    // the block's job number i (job + i*per_xcd < job_end)
    auto decode = [&](uint32_t i) {
        if (i - chunk_base >= 64u) refill(i);  // block-uniform
        const int L = (int)(i - chunk_base);
        const uint32_t erc = (uint32_t)__builtin_amdgcn_readlane((int)d_erc, L);
        Job j;
        j.e = erc & 0xffffu;
        j.row_count = (int)(erc >> 16);
        j.wexp = j.e < a.n_experts ? j.e : 0;
        j.col0 = (uint32_t)__builtin_amdgcn_readlane((int)d_col0, L);
        j.slot = (uint32_t)L;
        return j;
    };

    // per-lane routed-row indices of a job (from the row map): the
    // activation rows this thread stages and the rows of its finished
    // outputs (rows past row_count read the tile's first row: never stored)
    struct Rows {
        uint32_t x[XPER];
        uint32_t out[PER];
    };
    auto fetch_rows = [&](const Job& j) {
        const uint32_t* rj = rows_s + j.slot * BM;  // the job's entries, past row_count already the first
        Rows g;
#pragma unroll
        for (int jj = 0; jj < XPER; ++jj) g.x[jj] = rj[(tid + jj * THREADS) >> 5];
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int o = PER * b + p;
            g.out[p] = rj[4 * (o / (4 * C)) + o % 4];
        }
        return g;
    };

    const uint32_t x_div = a.layout == 1 ? 1u : a.top_k;  // routed row -> activation row
    // this thread's chunks of the activation tiles of two rounds: round g0
    // of the rows r0 (half 0) and round g1 of the rows r1 (half 1)
    auto load_x = [&](const uint32_t (&r0)[XPER], int g0, const uint32_t (&r1)[XPER], int g1) {
        XTile<2 * XPER> t;
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jj = 0; jj < XPER; ++jj) {
                const int chunk = (tid + jj * THREADS) & 31;
                const uint32_t xr = (h == 0 ? r0[jj] : r1[jj]) / x_div;
                const int g = h == 0 ? g0 : g1;
                const float* src = a.input + (size_t)xr * a.k + g * kRoundK + chunk * 4;
                if constexpr (TAIL) src -= g == last && chunk * 4 >= tail ? kRoundK : 0;  // zeroed in store_x
                t.v[h * XPER + jj] = *reinterpret_cast<const f32x4*>(src);
            }
        return t;
    };
    // publish them to LDS buffer `buf` (rounds g0, g1 in halves 0 and 1)
    auto store_x = [&](int buf, const XTile<2 * XPER>& t, int g0, int g1) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
#pragma unroll
            for (int jj = 0; jj < XPER; ++jj) {
                const int id = tid + jj * THREADS;
                const int lr = id >> 5, chunk = id & 31;
                float* dst = xs + ((size_t)(2 * buf + h) * BM + lr) * kRoundK + swz(lr, chunk) * 4;
                f32x4 v = t.v[h * XPER + jj];
                if constexpr (TAIL)
                    if ((h == 0 ? g0 : g1) == last && chunk * 4 >= tail) v = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
                *reinterpret_cast<f32x4*>(dst) = v;
            }
    };
    // piece i of this lane's granule lies past k in the last round (TAIL)
    auto w_past = [&](int i) { return b * kGranule + i * (16 / S) >= tail; };
    // this lane's weight granules of round g (columns past n read column n-1).
    // A load's address is a wavefront-uniform base (expert, the column group's
    // first column and the round, in scalar registers) plus a 32-bit lane
    // offset below 4*k*S + 1024 (the launch keeps that under 4 GB), so the
    // steady loop spends no vector instructions on 64-bit addresses, whatever
    // the size of an expert's matrix.
    const int wave_u = __builtin_amdgcn_readfirstlane(wave);
    auto fetch_w = [&](const Job& j, int g, WeightRound<DT, C>& wr) {
        const uint8_t* base = static_cast<const uint8_t*>(a.weights) + (size_t)j.wexp * a.stride;
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int c0 = min((int)j.col0 + wave_u * 4 * C + 4 * c, n - 1);  // uniform
            const int col = min((int)j.col0 + wave_u * 4 * C + 4 * c + q, n - 1);
            // the base sits one round back, so a TAIL piece loaded from the
            // previous round (zeroed in step2) keeps a non-negative offset
            const uint8_t* rb = base + (size_t)c0 * a.k * S + (size_t)(g - 1) * kRoundK * S;
            const uint32_t off = (uint32_t)(col - c0) * (uint32_t)a.k * (uint32_t)S + (uint32_t)(b * kGranule * S);
#pragma unroll
            for (int i = 0; i < Pieces<DT>::value; ++i) {
                const bool back = TAIL && g == last && w_past(i);
                const uint32_t o = off + 16u * (uint32_t)i + (back ? 0u : (uint32_t)(kRoundK * S));
                wr.p[c][i] = *reinterpret_cast<const u32x4*>(rb + o);
            }
        }
    };

    f32x4 acc[R][C];
#pragma unroll
    for (int r = 0; r < R; ++r)
#pragma unroll
        for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

    // one round from LDS tile `tile` (= 2*buffer + half) for row groups
    // R0 .. R0 + R/2 - 1 of the tile (each accumulator still takes its k
    // elements in order)
    auto compute_rows = [&](int tile, const float (&w)[C][kGranule], auto r0) __attribute__((always_inline)) {
        constexpr int R0 = decltype(r0)::value, RN = R / 2;
        const float* xb = xs + (size_t)tile * BM * kRoundK;
#pragma unroll
        for (int pr = 0; pr < 4; ++pr) {
            float2 xa[RN];
#pragma unroll
            for (int r = 0; r < RN; ++r) {
                const int row = 4 * (R0 + r) + q;
                const int chunk = swz(row, 2 * b + (pr >> 1));
                xa[r] = *reinterpret_cast<const float2*>(xb + row * kRoundK + chunk * 4 + (pr & 1) * 2);
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int r = 0; r < RN; ++r) {
                    const float xv = i == 0 ? xa[r].x : xa[r].y;
#pragma unroll
                    for (int c = 0; c < C; ++c) acc[R0 + r][c] = mfma_step(xv, w[c][2 * pr + i], acc[R0 + r][c]);
                }
        }
    };


    // slice sums (recursive halving over lane bits 5, 4, 3, 2, as in
    // grouped_kernel) and the stores of one finished job
    auto finish = [&](const Job& j, const Rows& g) {
        float val[NV];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int v = 0; v < 4; ++v) val[(r * C + c) * 4 + v] = acc[r][c][v];
        halving_exchange<NV>(val, lane);
        const bool nan_rows = j.e == a.n_experts;
#pragma unroll
        for (int p = 0; p < PER; ++p) {
            const int o = PER * b + p;
            const int r = o / (4 * C), c = (o / 4) % C, v = o % 4;
            const int lr = 4 * r + v;
            const int col = (int)j.col0 + wave * 4 * C + 4 * c + q;
            if (lr < j.row_count && col < n)
                a.output[(size_t)g.out[p] * a.n + col] = nan_rows ? quiet_nan() : val[p];
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    };

    // Two job slots, used alternately (static indices: loads in flight are
    // never copied between registers): while slot c's job runs, slot 1-c
    // holds the next job, whose row indices are already in flight.  The
    // block's job count is known up front, so the job loop has one exit.
    const uint32_t my_jobs = (job_end - job + per_xcd - 1) / per_xcd;
    Job jobs[2];
    Rows rws[2];
    uint32_t next = job + per_xcd, next_i = 1;
    jobs[0] = decode(0);
    rws[0] = fetch_rows(jobs[0]);
    jobs[1] = next < job_end ? decode(next_i) : jobs[0];
    rws[1] = fetch_rows(jobs[1]);

    // A step is two rounds: the weights of its rounds sit in register slots
    // 0 and 1, its activations in one LDS buffer (two rounds), so one
    // barrier serves two rounds.  During a step the next step's
    // activations and weights are requested.
    WeightRound<DT, C> ring[2];
    int buf = 0;
    {
        const XTile<2 * XPER> t = load_x(rws[0].x, 0, rws[0].x, 1);
        fetch_w(jobs[0], 0, ring[0]);
        fetch_w(jobs[0], 1, ring[1]);
        store_x(0, t, 0, 1);
    }
    __syncthreads();

    // One step from LDS buffer `buf`: request the next step's activations
    // (round gx0 of the rows xr0, round gx1 of the rows xr1), then per round
    // h widen its weights, refill slot h with round gw0 of job j0 (h = 0) or
    // gw1 of job j1 (h = 1) and compute; publish the activations to the other
    // buffer.  up0, up1: the tile of round h has rows in its upper half of
    // row groups (uniform).  mid() runs between the two rounds.  LAST (bit h):
    // round h is its job's last round (TAIL: its pieces past k become zeros).
    auto step2 = [&](const uint32_t (&xr0)[XPER], int gx0, const uint32_t (&xr1)[XPER], int gx1,
                     const Job& j0, int gw0, const Job& j1, int gw1, bool up0, bool up1,
                     auto mid, auto lastc) __attribute__((always_inline)) {
        constexpr int LAST = decltype(lastc)::value;
        const XTile<2 * XPER> t = load_x(xr0, gx0, xr1, gx1);
        __builtin_amdgcn_sched_barrier(0);
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            if (TAIL && ((LAST >> h) & 1)) {  // h is a constant after unrolling
#pragma unroll
                for (int c = 0; c < C; ++c)
#pragma unroll
                    for (int i = 0; i < Pieces<DT>::value; ++i)
                        if (w_past(i)) ring[h].p[c][i] = u32x4{0u, 0u, 0u, 0u};
            }
            float w[C][kGranule];
            widen_w_pieces_all<DT, C>(ring[h], w);
            __builtin_amdgcn_sched_barrier(0);
            fetch_w(h == 0 ? j0 : j1, h == 0 ? gw0 : gw1, ring[h]);
            __builtin_amdgcn_sched_barrier(0);
            compute_rows(2 * buf + h, w, IntC<0>{});
            if (h == 0 ? up0 : up1) compute_rows(2 * buf + h, w, IntC<R / 2>{});
            __builtin_amdgcn_sched_barrier(0);
            if (h == 0) {
                mid();
                __builtin_amdgcn_sched_barrier(0);
            }
        }
        store_x(buf ^ 1, t, gx0, gx1);
        __syncthreads();
        buf ^= 1;
    };
    // the usual step: rounds gx, gx+1 of the rows xrows, rounds gw, gw+1 of
    // job j (LAST as in step2)
    auto step = [&](const uint32_t (&xrows)[XPER], int gx, const Job& j, int gw, bool upper,
                    auto lastc) __attribute__((always_inline)) {
        step2(xrows, gx, xrows, gx + 1, j, gw, j, gw + 1, upper, upper, [] {}, lastc);
    };
    // the job in slot c; afterwards slot c takes the job after next (or
    // repeats slot 1-c's job when there is none: its loads stay in bounds,
    // its results unused).  With an even number of rounds every job starts
    // on a step.  With an odd number (at least three) the jobs of slot 0
    // start on a step and the jobs of slot 1 one round later: a slot-0 job's
    // last round and the next job's first share a step, with the slot-0 job
    // finished between them, so the stream of steps has no gap.
    auto run_job = [&](auto cc) __attribute__((always_inline)) {
        constexpr int c = decltype(cc)::value, o = 1 - c;
        // LAST flags for the steps holding a job's last round (only TAIL uses
        // them; without a tail every step is the same instantiation)
        constexpr int kLast0 = TAIL ? 1 : 0, kLast1 = TAIL ? 2 : 0;
        // An expert's last row tile with at most 2R rows skips the steps of
        // the upper half of its row groups (their outputs are never stored;
        // the others keep their order).  One uniform branch per round does
        // it, so every job runs the same loop: separate loops per row count
        // cost more in register copies at their entries than they saved.
        const bool upper = __builtin_amdgcn_readfirstlane(jobs[c].row_count) > 4 * (R / 2);
        if constexpr (!ODD) {
            int g = 0;
            for (; g + 2 < rounds; g += 2) step(rws[c].x, g + 2, jobs[c], g + 2, upper, IntC<0>{});
            step(rws[o].x, 0, jobs[o], 0, upper, IntC<kLast1>{});
            finish(jobs[c], rws[c]);
        } else if constexpr (c == 0) {
            // rounds 0 .. rounds-2 in pairs; the last pair requests this
            // job's last round and slot 1's first
            int g = 0;
            for (; g + 3 < rounds; g += 2) step(rws[0].x, g + 2, jobs[0], g + 2, upper, IntC<0>{});
            step2(rws[0].x, rounds - 1, rws[1].x, 0, jobs[0], rounds - 1, jobs[1], 0, upper, upper, [] {},
                  IntC<0>{});
            // the shared step: this job's last round, then slot 1's round 0
            const bool upper1 = __builtin_amdgcn_readfirstlane(jobs[1].row_count) > 4 * (R / 2);
            step2(rws[1].x, 1, rws[1].x, 2, jobs[1], 1, jobs[1], 2, upper, upper1,
                  [&] { finish(jobs[0], rws[0]); }, IntC<kLast0>{});
        } else {
            // round 0 is done: rounds 1 .. rounds-1 in pairs, the last one
            // requesting slot 0's first two
            int g = 1;
            for (; g + 3 < rounds; g += 2) step(rws[1].x, g + 2, jobs[1], g + 2, upper, IntC<0>{});
            step(rws[0].x, 0, jobs[0], 0, upper, IntC<kLast1>{});
            finish(jobs[1], rws[1]);
        }
        next += per_xcd;
        ++next_i;
        jobs[c] = next < job_end ? decode(next_i) : jobs[o];
        rws[c] = fetch_rows(jobs[c]);
    };
    uint32_t i = 0;
    for (; i + 2 <= my_jobs; i += 2) {
        run_job(IntC<0>{});
        run_job(IntC<1>{});
    }
    if (i < my_jobs) run_job(IntC<0>{});
}

template <int DT, int R, int C, int WAVES>
hipError_t launch_cfg(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                      hipStream_t stream) {
    constexpr uint32_t BM = 4 * R, BN = 4 * C * WAVES;
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t ntiles = (a.n + BN - 1) / BN;
    // every bucket adds at most one partial row tile
    const uint64_t job_bound = (routed / BM + a.n_experts + 1) * ntiles;
    // the streamed form needs vector rows, two or more rounds (three or more
    // when their number is odd) and 4 weight rows within 32-bit lane offsets
    const uint32_t rounds = (a.k + kRoundK - 1) / kRoundK;
    const bool odd = rounds % 2 == 1, tail = a.k % kRoundK != 0;
    const bool stream_form = a.vec && rounds >= (odd ? 3u : 2u) &&
                             4ull * a.k * DtypeSize<DT>::value + 1024 <= 0xffffffffull;
    auto kernel = !stream_form ? grouped_kernel<DT, R, C, WAVES>
                  : odd ? (tail ? grouped_stream_kernel<DT, R, C, WAVES, true, true>
                                : grouped_stream_kernel<DT, R, C, WAVES, true, false>)
                        : (tail ? grouped_stream_kernel<DT, R, C, WAVES, false, true>
                                : grouped_stream_kernel<DT, R, C, WAVES, false, false>);
    const size_t table = stream_form ? (3 * (size_t)a.n_experts + 4 + 64 * BM) : (a.n_experts + 2);
    const size_t lds = (stream_form ? 4 : 2) * BM * kRoundK * sizeof(float) + table * sizeof(uint32_t);
    int per_cu = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kernel, 64 * WAVES, lds) != hipSuccess ||
        per_cu < 1)
        per_cu = 1;
    const uint64_t resident = (uint64_t)(device_cus > 0 ? device_cus : 256) * per_cu;
    uint64_t grid = job_bound < resident ? job_bound : resident;
    grid = (grid + kXcds - 1) / kXcds * kXcds;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(64 * WAVES), lds, stream, a, buf.counts,
                       buf.offsets, buf.rows);
    return launched(stream_form ? EIDM_KERNEL_GROUPED_STREAM : EIDM_KERNEL_GROUPED_JOB, (uint32_t)grid, 64 * WAVES,
                    (uint32_t)lds);
}

// Tile shape per weight type.  16-bit weights: BM = 16 rows x BN = 128
// columns (small row tiles waste few rows in an expert's last tile); f32
// weights need twice the registers per weight round, so they take R = 8,
// C = 2 (32 x 64 tiles) to stay within 256 VGPRs.
template <int DT>
hipError_t launch_dt(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                     hipStream_t stream) {
    if constexpr (DT == kDtypeF32)
        return launch_cfg<DT, 8, 2, 8>(a, buf, device_cus, stream);
    else
        return launch_cfg<DT, EIDM_GROUPED_R, EIDM_GROUPED_C, EIDM_GROUPED_WAVES>(a, buf, device_cus, stream);
}

}  // namespace

hipError_t launch_grouped(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                          hipStream_t stream) {
    if (grouped16_supported(a)) return launch_grouped16(a, buf, device_cus, stream);
    switch (a.dtype) {
    case kDtypeF32: return launch_dt<kDtypeF32>(a, buf, device_cus, stream);
    case kDtypeF16: return launch_dt<kDtypeF16>(a, buf, device_cus, stream);
    case kDtypeBF16: return launch_dt<kDtypeBF16>(a, buf, device_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace eidm
