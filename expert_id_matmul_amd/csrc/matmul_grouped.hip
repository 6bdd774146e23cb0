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
// k-slices, and within a block the 4 A-rows are 4 gathered routed rows and
// the 4 B-columns are 4 output columns, so one step advances 16 outputs of
// every slice at once.  A wavefront holds a (4R rows) x (4C columns) tile;
// a block is 2x2 wavefronts.
//
// Tile jobs are numbered expert-major (bucket e, column tile nt, row tile
// mt), with the row tile fastest so the jobs that share an expert's weight
// columns run together; every block walks the numbering with a grid stride.
// The job count comes from the map's per-expert counts, which each block
// reads and scans itself.  The last bucket (ids >= n_experts) gets quiet NaN
// rows.
#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

constexpr int kGroupedThreads = 256;

template <int DT, int R, int C>
__global__ __launch_bounds__(kGroupedThreads) void grouped_kernel(MatmulArgs a,
                                                                  const uint32_t* __restrict__ counts,
                                                                  const uint32_t* __restrict__ offsets,
                                                                  const uint32_t* __restrict__ rows) {
    constexpr int S = DtypeSize<DT>::value;
    constexpr int BM = 8 * R, BN = 8 * C;  // 2x2 wavefronts of (4R x 4C)
    extern __shared__ uint32_t job_start[];  // [buckets + 1]
    __shared__ uint32_t wave_tot[4];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int b = lane >> 2, q = lane & 3;
    const int wr = wave >> 1, wc = wave & 1;
    const uint32_t buckets = a.n_experts + 1;
    const uint32_t ntiles = (a.n + BN - 1) / BN;
    const int n = (int)a.n, k = (int)a.k;

    // jobs per bucket -> exclusive prefix in LDS
    {
        const uint32_t per = (buckets + kGroupedThreads - 1) / kGroupedThreads;
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
        for (int w = 0; w < 4; ++w) {
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
    const bool vec = a.vec;

    for (uint32_t job = blockIdx.x; job < total_jobs; job += gridDim.x) {
        // bucket of this job: last e with job_start[e] <= job
        uint32_t lo = 0, hi = buckets;  // invariant: job_start[lo] <= job < job_start[hi]
        while (hi - lo > 1) {
            const uint32_t mid = (lo + hi) >> 1;
            if (job_start[mid] <= job) lo = mid; else hi = mid;
        }
        const uint32_t e = lo;
        const uint32_t local = job - job_start[e];
        const uint32_t mtiles = (counts[e] + BM - 1) / BM;
        const uint32_t nt = local / mtiles, mt = local % mtiles;
        const uint32_t row_begin = offsets[e] + mt * BM;
        const int row_count = (int)min((uint32_t)BM, counts[e] - mt * BM);
        const int col_base = (int)(nt * BN) + wc * 4 * C;
        const int row_base = wr * 4 * R;  // within the tile

        if (e == a.n_experts) {  // ids naming no expert: NaN rows
            for (int i = lane; i < 4 * R * 4 * C; i += 64) {
                const int lr = row_base + i / (4 * C), col = col_base + i % (4 * C);
                if (lr < row_count && col < n)
                    a.output[(size_t)rows[row_begin + lr] * a.n + col] = quiet_nan();
            }
            continue;
        }

        // A operand rows: lane q feeds row 4r+q of each row group r
        const float* xrow[R];
        bool rvalid[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int lr = row_base + 4 * r + q;
            rvalid[r] = lr < row_count;
            uint32_t xr = 0;
            if (rvalid[r]) {
                const uint32_t rho = rows[row_begin + lr];
                xr = a.layout == 1 ? rho : rho / a.top_k;
            }
            xrow[r] = a.input + (size_t)xr * a.k;
        }
        // B operand columns: lane q feeds column 4c+q of each column group c
        const uint8_t* wexp = static_cast<const uint8_t*>(a.weights) + (size_t)e * a.stride;
        const uint8_t* wrow[C];
        bool cvalid[C];
#pragma unroll
        for (int c = 0; c < C; ++c) {
            const int col = col_base + 4 * c + q;
            cvalid[c] = col < n;
            wrow[c] = wexp + (size_t)(cvalid[c] ? col : 0) * a.k * S;
        }

        f32x4 acc[R][C];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c) acc[r][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};

        for (int g = 0; g < rounds; ++g) {
            const int kk = g * kRoundK + b * kGranule;
            float x[R][kGranule];
            float w[C][kGranule];
#pragma unroll
            for (int r = 0; r < R; ++r) load_input_granule(xrow[r], kk, k, rvalid[r], vec, x[r]);
#pragma unroll
            for (int c = 0; c < C; ++c) load_weight_granule<DT>(wrow[c], kk, k, cvalid[c], vec, w[c]);
#pragma unroll
            for (int i = 0; i < kGranule; ++i)
#pragma unroll
                for (int r = 0; r < R; ++r)
#pragma unroll
                    for (int c = 0; c < C; ++c) acc[r][c] = mfma_step(x[r][i], w[c][i], acc[r][c]);
        }

        // slice totals; lanes of slice b < 4 write output row 4r+b, column 4c+q
        uint32_t out_row[R];
        bool out_valid[R];
#pragma unroll
        for (int r = 0; r < R; ++r) {
            const int lr = row_base + 4 * r + (b & 3);
            out_valid[r] = b < 4 && lr < row_count;
            out_row[r] = out_valid[r] ? rows[row_begin + lr] : 0;
        }
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
            for (int c = 0; c < C; ++c) {
                float t[4];
#pragma unroll
                for (int v = 0; v < 4; ++v) t[v] = slice_tree(acc[r][c][v]);
                const float mine = b == 0 ? t[0] : b == 1 ? t[1] : b == 2 ? t[2] : t[3];
                const int col = col_base + 4 * c + q;
                if (out_valid[r] && col < n) a.output[(size_t)out_row[r] * a.n + col] = mine;
            }
    }
}

template <int DT, int R, int C>
hipError_t launch_cfg(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                      hipStream_t stream) {
    constexpr uint32_t BM = 8 * R, BN = 8 * C;
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t ntiles = (a.n + BN - 1) / BN;
    // every bucket adds at most one partial row tile
    const uint64_t job_bound = (routed / BM + a.n_experts + 1) * ntiles;
    const uint64_t resident = (uint64_t)(device_cus > 0 ? device_cus : 256) * 2;
    const uint32_t grid = (uint32_t)(job_bound < resident ? job_bound : resident);
    const size_t lds = (a.n_experts + 2) * sizeof(uint32_t);
    hipLaunchKernelGGL((grouped_kernel<DT, R, C>), dim3(grid), dim3(kGroupedThreads), lds, stream,
                       a, buf.counts, buf.offsets, buf.rows);
    return hipGetLastError();
}

template <int DT>
hipError_t launch_dt(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                     hipStream_t stream) {
    return launch_cfg<DT, 4, 4>(a, buf, device_cus, stream);
}

}  // namespace

hipError_t launch_grouped(const MatmulArgs& a, const MapBuffers& buf, int device_cus,
                          hipStream_t stream) {
    switch (a.dtype) {
    case kDtypeF32: return launch_dt<kDtypeF32>(a, buf, device_cus, stream);
    case kDtypeF16: return launch_dt<kDtypeF16>(a, buf, device_cus, stream);
    case kDtypeBF16: return launch_dt<kDtypeBF16>(a, buf, device_cus, stream);
    default: return hipErrorInvalidValue;
    }
}

}  // namespace eidm
