// grouped16_kernel.hpp -- the 16x16x1 Grouped kernel for 16-bit weights and
// its launch.  Two sources build it: one keeps the matrix-core accumulators
// in the architectural registers, the other in the accumulation registers
// (a per-source compiler setting); each gets its own copies (an unnamed
// namespace).
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs: fn expected_dispatches
// gives the grouped route a map dispatch and then tiles of (rows of one
// expert) x (output columns); the value-independence theorem statement
// requires it to reproduce the Direct route's bits, differing only in which
// independent rows are computed together.
//
// The canonical order (eidm_device.hpp) is kept: 16 slices, granule g of 8
// consecutive k belongs to slice g mod 16, each slice an ascending chain of
// single-rounding fmas from +0, the slice sums paired (s, s^8), (s, s^4),
// (s, s^2), (s, s^1).  The step is v_mfma_f32_16x16x1_4b_f32: 4 independent
// 16x16 blocks with one product per output (it returns fma(a, b, c) bit for
// bit, measured on gfx950 over every operand class).  Operand lane 16*blk + i
// feeds row i (A) and column i (B) of block blk; result register 4*blk + v of
// lane l holds row 4*(l/16) + v, column l%16 of block blk.  The slices are
// the 4 blocks times 4 register sets: slice s = 4*set + blk.  So every slice
// sum of an output lives in the registers of one lane, and the pairing at the
// end is 15 lane-local adds per output, with no cross-lane traffic.
//
// Tiles: a job is 32 gathered rows of one expert (two 16-row tiles) by 64
// output columns; a block of 4 wavefronts (one per SIMD) takes 16 columns
// each.  Per round of 128 k a wavefront issues 4 sets x 8 k x 2 row tiles =
// 64 steps on one 16-byte weight load and 8 widenings per set.  Vector ALU
// instructions do not overlap the matrix core on this chip (a probe: each
// costs about 6 cycles of matrix-core time, from any wavefront of the SIMD),
// so the layout keeps them to about one per two steps.
//
// Pipeline (one barrier per round): the activation tile of a round (32 rows
// x 128 f32, rows padded to 528 bytes so the 16 rows read together fall in
// 16 different bank groups) goes through one of three LDS buffers; the
// weights go straight into a two-round register ring, one 16-byte slot per
// set.  Round p computes from buffer p%3, reads the first operands of round
// p+1 from buffer (p+1)%3 (published a round earlier), and stages round p+2
// into buffer (p+2)%3 (free since the barrier that ended round p-1).  Loads
// run two rounds ahead across job boundaries: the rounds of all the jobs a
// block walks are one stream.
#pragma once

#include <atomic>

#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {
namespace {

typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef unsigned int g16u32x4 __attribute__((ext_vector_type(4)));

template <int V> struct IntC2 { static constexpr int value = V; };
template <bool V> struct BoolC2 { static constexpr bool value = V; };

constexpr int kG16Xcds = 8;
constexpr int kG16Waves = 4;
constexpr int kG16Threads = 64 * kG16Waves;
constexpr int kG16BM = 32;                        // gathered rows per job
constexpr int kG16WN = 16;                        // output columns per wavefront
constexpr int kG16BN = kG16WN * kG16Waves;        // output columns per job
constexpr int kG16RowBytes = kRoundK * 4 + 16;    // one activation row of a round, padded
constexpr int kG16XBuf = kG16BM * kG16RowBytes;   // one round's activation tile
constexpr int kG16XBufs = 3;
constexpr int kG16Chunk = 64;                     // jobs decoded together
constexpr int kG16Ent = kG16Chunk * kG16BM;       // row-table entries per chunk
constexpr int kG16Stage = kG16BM * (kRoundK / 4) / kG16Threads;  // 16-byte chunks staged per thread per round
static_assert(kG16Stage == 4, "staging layout assumes 4 chunks per thread");

template <int DT>
__device__ __forceinline__ void g16_widen8(const g16u32x4& p, float (&w)[8]) {
    widen_pair<DT>(p.x, w[0], w[1]);
    widen_pair<DT>(p.y, w[2], w[3]);
    widen_pair<DT>(p.z, w[4], w[5]);
    widen_pair<DT>(p.w, w[6], w[7]);
}

// Keeps the loads issued before it where they are: no memory access moves
// across (an empty asm statement that clobbers memory); arithmetic still can.
__device__ __forceinline__ void g16_pin() { asm volatile("" ::: "memory"); }

__device__ __forceinline__ f32x16 g16_step(float a, float b, f32x16 acc) {
    return __builtin_amdgcn_mfma_f32_16x16x1f32(a, b, acc, 0, 0, 0);
}

// Job of a block's walk: bucket e (n_experts: ids naming no expert), rows in
// the tile, first output column, and its slot in the row tables.
struct G16Job {
    uint32_t e, rc, col0, slot;
};

template <int DT, bool ODD, bool TAIL>
__global__ __launch_bounds__(kG16Threads, 1) void grouped16_kernel(MatmulArgs a,
                                                                    const uint32_t* __restrict__ counts,
                                                                    const uint32_t* __restrict__ offsets,
                                                                    const uint32_t* __restrict__ rows) {
    static_assert(DtypeSize<DT>::value == 2, "16-bit weights");
    const uint32_t buckets = a.n_experts + 1;
    extern __shared__ __align__(16) uint8_t smem[];
    uint8_t* xs = smem;                                                                // [3][32][528 B]
    uint32_t* xoff_s = reinterpret_cast<uint32_t*>(smem + kG16XBufs * kG16XBuf);       // [2][64][32] input byte offsets
    uint32_t* yoff_s = xoff_s + 2 * kG16Ent;                                           // [2][64][32] output row offsets
    uint32_t* job_start = yoff_s + 2 * kG16Ent;                                        // [buckets+1]
    uint32_t* cnt_s = job_start + buckets + 1;                                         // [buckets]
    uint32_t* off_s = cnt_s + buckets;                                                 // [buckets]
    __shared__ uint32_t wave_tot[kG16Waves];

    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int blk = lane >> 4, l16 = lane & 15;
    const int srow = tid >> 5, schunk = tid & 31;  // staging: rows srow + 8*jj, 16-byte chunk schunk
    const uint32_t ntiles = (a.n + kG16BN - 1) / kG16BN;
    const int n = (int)a.n, k = (int)a.k;
    const int R = (k + kRoundK - 1) / kRoundK;  // rounds per job (at least 3)
    const int tail = k - (R - 1) * kRoundK;     // elements of the last round inside k

    // ---- job table: jobs per bucket -> exclusive prefix, with counts and
    // offsets.  A job's cost is its number of 16-row tiles (the matrix-core
    // work: a job of at most 16 rows skips its second tile), so bucket e
    // costs ceil(count/16) x ntiles.  The job list is cut into one share per
    // XCD of equal cost: share x starts at the first job whose cost prefix
    // reaches x/8 of the total.
    __shared__ uint32_t cost_tot[kG16Waves], share_s[kG16Xcds + 1];
    {
        const uint32_t per = (buckets + kG16Threads - 1) / kG16Threads;
        const uint32_t begin = min(buckets, (uint32_t)tid * per);
        const uint32_t end = min(buckets, begin + per);
        uint32_t s = 0, cs = 0;
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t c = counts[i];
            cnt_s[i] = c;
            off_s[i] = offsets[i];
            const uint32_t jobs = ((c + kG16BM - 1) / kG16BM) * ntiles;
            job_start[i] = jobs;
            s += jobs;
            cs += ((c + 15) / 16) * ntiles;
        }
        uint32_t inc = s, cinc = cs;
#pragma unroll
        for (int d = 1; d < 64; d <<= 1) {
            const uint32_t o = __shfl_up(inc, d), co = __shfl_up(cinc, d);
            if (lane >= d) {
                inc += o;
                cinc += co;
            }
        }
        if (lane == 63) {
            wave_tot[wave] = inc;
            cost_tot[wave] = cinc;
        }
        __syncthreads();
        uint32_t run = inc - s, total = 0, crun = cinc - cs, ctotal = 0;
        for (int w = 0; w < kG16Waves; ++w) {
            if (w < wave) {
                run += wave_tot[w];
                crun += cost_tot[w];
            }
            total += wave_tot[w];
            ctotal += cost_tot[w];
        }
        for (uint32_t i = begin; i < end; ++i) {
            const uint32_t v = job_start[i];
            job_start[i] = run;
            // the XCD cuts that fall in this bucket's cost span [crun, crun + cost)
            const uint32_t c = cnt_s[i];
            const uint32_t cost = ((c + 15) / 16) * ntiles;
            for (uint32_t x = 1; x < (uint32_t)kG16Xcds; ++x) {
                const uint32_t th = (uint32_t)((uint64_t)x * ctotal / kG16Xcds);
                if (th < crun || th >= crun + cost) continue;
                // job l of the bucket starts at cost 2l up to its last row tile,
                // whose jobs cost 1 or 2 each
                const uint32_t d = th - crun;
                const uint32_t full2 = 2u * (c / kG16BM) * ntiles;
                const uint32_t wl = c % kG16BM > 16 ? 2u : 1u;
                const uint32_t l = d <= full2 ? (d + 1) / 2 : full2 / 2 + (d - full2 + wl - 1) / wl;
                share_s[x] = run + l;
            }
            run += v;
            crun += cost;
        }
        if (tid == 0) {
            job_start[buckets] = total;
            share_s[0] = 0;
            share_s[kG16Xcds] = total;
            if (ctotal == 0)
                for (int x = 1; x < kG16Xcds; ++x) share_s[x] = total;
        }
        __syncthreads();
    }
    const uint32_t total_jobs = job_start[buckets];
    // Each XCD walks its share of the job list with its blocks side by side
    // (the hardware deals blocks to the XCDs round-robin), so the column
    // tiles of one expert's row tile meet in one L2.
    const uint32_t per_xcd = gridDim.x / kG16Xcds;
    const uint32_t xcd = blockIdx.x % kG16Xcds;
    const uint32_t job0 = share_s[xcd] + blockIdx.x / kG16Xcds;
    const uint32_t job_end = min(total_jobs, share_s[xcd + 1]);
    if (job0 >= job_end) return;  // the whole block leaves together
    const uint32_t my_jobs = (job_end - job0 + per_xcd - 1) / per_xcd;

    // ---- job descriptors, 64 at a time: lane L of every wavefront holds job
    // base + L of a chunk (bucket | rows << 16, first column), for the
    // current and the previous chunk; the same pass writes the chunk's input
    // and output row offsets into LDS table (chunk number & 1), so a job's
    // row data are LDS reads.  Only the load side, which runs at most two jobs
    // ahead of the compute side, moves to a new chunk.
    uint32_t top = 1;
    while (top * 2 <= buckets) top *= 2;
    uint32_t chunk_base = 0x80000000u;
    uint32_t d_erc[2] = {0, 0}, d_col0[2] = {0, 0};  // by chunk parity
    const uint32_t x_div = a.layout == 1 ? 1u : a.top_k;
    auto refill = [&](uint32_t i0) {
        chunk_base = i0;
        const uint32_t par = (i0 / kG16Chunk) & 1u;
        const uint32_t tbl = par * kG16Ent;
        uint32_t d_rb = 0, erc = 0, col0 = 0;
        const uint64_t jb64 = (uint64_t)job0 + ((uint64_t)i0 + (uint64_t)lane) * per_xcd;
        if (jb64 < job_end) {
            const uint32_t jb = (uint32_t)jb64;
            uint32_t e = 0;
            for (uint32_t st = top; st; st >>= 1)
                if (e + st < buckets && job_start[e + st] <= jb) e += st;
            const uint32_t local = jb - job_start[e];
            const uint32_t mt = local / ntiles, nt = local - mt * ntiles;
            erc = e | (min((uint32_t)kG16BM, cnt_s[e] - mt * kG16BM) << 16);
            col0 = nt * kG16BN;
            d_rb = off_s[e] + mt * kG16BM;
        }
        if (par) { d_erc[1] = erc; d_col0[1] = col0; } else { d_erc[0] = erc; d_col0[0] = col0; }
        constexpr int EPT = kG16Ent / kG16Threads;
        uint32_t v[EPT];
#pragma unroll
        for (int jj = 0; jj < EPT; ++jj) {
            const int ent = tid + jj * kG16Threads;
            const int L = ent / kG16BM, lr = ent % kG16BM;
            const uint32_t rb = (uint32_t)__shfl((int)d_rb, L);
            const uint32_t rc = (uint32_t)__shfl((int)erc, L) >> 16;
            v[jj] = rows[rb + ((uint32_t)lr < rc ? (uint32_t)lr : 0u)];  // rows past rc repeat the first
        }
#pragma unroll
        for (int jj = 0; jj < EPT; ++jj) {
            const int ent = tid + jj * kG16Threads;
            xoff_s[tbl + ent] = (v[jj] / x_div) * (uint32_t)k * 4u;
            yoff_s[tbl + ent] = v[jj] * (uint32_t)n;
        }
        __syncthreads();
    };
    auto decode = [&](uint32_t i) {
        // block-uniform; only the load side reaches a new chunk (the compute
        // side's jobs are in the current or the previous one)
        if (chunk_base == 0x80000000u || i >= chunk_base + (uint32_t)kG16Chunk) refill(i - i % kG16Chunk);
        const uint32_t par = (i / kG16Chunk) & 1u;
        const int L = (int)(i % kG16Chunk);
        const uint32_t erc = (uint32_t)__builtin_amdgcn_readlane((int)(par ? d_erc[1] : d_erc[0]), L);
        G16Job j;
        j.e = erc & 0xffffu;
        j.rc = erc >> 16;
        j.col0 = (uint32_t)__builtin_amdgcn_readlane((int)(par ? d_col0[1] : d_col0[0]), L);
        j.slot = par * kG16Ent + (uint32_t)L * kG16BM;
        return j;
    };

    // ---- load side: state of the job whose rounds are loaded now (0) and of
    // the one after it (1)
    struct LoadState {
        const uint8_t* w;           // the expert's weights (block-uniform)
        uint32_t woff;              // this lane's weight column + granule offset
        uint32_t xoff[kG16Stage];   // this thread's staged input chunks
    };
    auto load_state = [&](const G16Job& j) {
        LoadState st;
        const uint32_t wexp = j.e < a.n_experts ? j.e : 0u;
        st.w = static_cast<const uint8_t*>(a.weights) + (size_t)wexp * a.stride;
        const int col = min((int)j.col0 + wave * kG16WN + l16, n - 1);
        st.woff = (uint32_t)col * (uint32_t)k * 2u + (uint32_t)blk * 16u;
#pragma unroll
        for (int jj = 0; jj < kG16Stage; ++jj)
            st.xoff[jj] = xoff_s[j.slot + srow + 8 * jj] + (uint32_t)schunk * 16u;
        return st;
    };
    // TAIL: pieces of the last round past k are loaded one round earlier
    // (in bounds) and replaced by zeros where they are used.
    auto w_past = [&](int set) { return TAIL && 32 * set + 8 * blk >= tail; };
    const bool x_past = TAIL && 4 * schunk >= tail;

    const uint8_t* const xin = reinterpret_cast<const uint8_t*>(a.input);
    auto load_x = [&](const LoadState& st, int lr, f32x4 (&stg)[kG16Stage]) {
        const uint8_t* base = xin + (size_t)lr * kRoundK * 4;
        const uint32_t back = (TAIL && lr == R - 1 && x_past) ? (uint32_t)kRoundK * 4u : 0u;
#pragma unroll
        for (int jj = 0; jj < kG16Stage; ++jj)
            stg[jj] = *reinterpret_cast<const f32x4*>(base + (size_t)st.xoff[jj] - (size_t)back);
    };
    auto load_w = [&](const LoadState& st, int lr, int set, g16u32x4& slot) {
        const uint8_t* base = st.w + (size_t)lr * kRoundK * 2;
        const uint32_t back = (TAIL && lr == R - 1 && w_past(set)) ? (uint32_t)kRoundK * 2u : 0u;
        slot = *reinterpret_cast<const g16u32x4*>(base + (size_t)st.woff + 64 * set - (size_t)back);
    };
    auto store_x = [&](int buf, int lr, const f32x4 (&stg)[kG16Stage]) {
        uint8_t* dst = xs + buf * kG16XBuf + srow * kG16RowBytes + schunk * 16;
        const bool zero = TAIL && lr == R - 1 && x_past;
#pragma unroll
        for (int jj = 0; jj < kG16Stage; ++jj)
            *reinterpret_cast<f32x4*>(dst + jj * 8 * kG16RowBytes) = zero ? f32x4{0.0f, 0.0f, 0.0f, 0.0f} : stg[jj];
    };
    // A operands of one set: rows l16 and 16 + l16, granule 4*set + blk (8 floats each)
    const int rd_lane = l16 * kG16RowBytes + blk * 32;
    auto read_a = [&](int buf, int set, f32x4 (&av)[2][2]) {
        const uint8_t* src = xs + buf * kG16XBuf + rd_lane + set * 128;
#pragma unroll
        for (int rt = 0; rt < 2; ++rt)
#pragma unroll
            for (int h = 0; h < 2; ++h)
                av[rt][h] = *reinterpret_cast<const f32x4*>(src + rt * 16 * kG16RowBytes + h * 16);
    };

    f32x16 acc[2][4];
    // slice sums in the canonical pairing, and the stores.  The eight output
    // rows' offsets are read from LDS first, so their latency is paid once;
    // each total is formed outside the store's branch.
    // TWO: the job has rows in its second 16-row tile (else that tile's
    // sums are not formed).
    auto finish = [&](const G16Job& j, auto twoc) __attribute__((always_inline)) {
        constexpr int NRT = decltype(twoc)::value ? 2 : 1;
        const int col = (int)j.col0 + wave * kG16WN + l16;
        const bool nan_rows = j.e == a.n_experts;
        const bool col_ok = col < n;
        uint32_t yo[2][4];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) yo[rt][v] = yoff_s[j.slot + 16 * rt + 4 * blk + v];
#pragma unroll
        for (int rt = 0; rt < NRT; ++rt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                float u[4];
#pragma unroll
                for (int bb = 0; bb < 4; ++bb) {
                    // slice 4*set + bb: (s, s^8) pairs sets 0-2 and 1-3, then (s, s^4)
                    const float t0 = acc[rt][0][4 * bb + v] + acc[rt][2][4 * bb + v];
                    const float t1 = acc[rt][1][4 * bb + v] + acc[rt][3][4 * bb + v];
                    u[bb] = t0 + t1;
                }
                // (s, s^2) pairs blocks 0-2 and 1-3, then (s, s^1)
                const float total = (u[0] + u[2]) + (u[1] + u[3]);
                if (col_ok && 16 * rt + 4 * blk + v < (int)j.rc)
                    a.output[(size_t)(yo[rt][v] + (uint32_t)col)] = nan_rows ? quiet_nan() : total;
            }
    };

    // ---- prologue: weights of rounds 0 and 1, activations of rounds 0, 1
    // and 2 of job 0 (the last stay staged in registers)
    LoadState Lc = load_state(decode(0));  // decode(0) also fills the first chunk
    g16u32x4 ring[2][4];
    f32x4 stg[kG16Stage];
    {
        f32x4 s0[kG16Stage], s1[kG16Stage];
        load_x(Lc, 0, s0);
#pragma unroll
        for (int s = 0; s < 4; ++s) load_w(Lc, 0, s, ring[0][s]);
        load_x(Lc, 1, s1);
#pragma unroll
        for (int s = 0; s < 4; ++s) load_w(Lc, 1, s, ring[1][s]);
        load_x(Lc, 2, stg);
        store_x(0, 0, s0);
        store_x(1, 1, s1);
    }
    __syncthreads();
    f32x4 av[2][2][2];  // [parity of the set][row tile][half]
    read_a(0, 0, av[0]);
    int bc = 0;  // LDS buffer of the compute position

    // Weights are widened one set ahead, so no matrix-core step waits on the
    // instruction that produced its operand (a widening placed right before
    // its step costs about three times as much as an independent one).  wc:
    // the widened weights of the set about to be computed.
    float wc[8];
    auto widen_slot = [&](const g16u32x4& r, int set, bool last, float (&w)[8]) {
        g16u32x4 raw = r;
        if (TAIL && last && w_past(set)) raw = g16u32x4{0u, 0u, 0u, 0u};
        g16_widen8<DT>(raw, w);
    };
    widen_slot(ring[0][0], 0, false, wc);

    // One round of the stream in register slot SL.  It computes its position
    // p, loads the weights of position p+2 (load state Lw, round lrw) and the
    // activations of position p+3 (Lx, lrx), and stores the staged
    // activations of position p+2 into LDS.  FIRST: the job's first round
    // (its chains start from +0).  TWO: the job has rows in its second 16-row
    // tile (otherwise those steps are skipped; their outputs are never
    // stored).  lastw: this round is its job's last; lastn: the next one is
    // (TAIL zeroes their weights past k).  Each set: read the next set's
    // operands from LDS, half of this set's steps, widen the next set's
    // weights and refill this set's weight slot, the other half.  At set 2
    // the staged activations go to LDS (done long before the barrier) and
    // the next ones are requested.
    auto round = [&](auto slotc, auto firstc, auto twoc, const LoadState& Lw, int lrw, const LoadState& Lx,
                     int lrx, bool lastw, bool lastn) __attribute__((always_inline)) {
        constexpr int SL = decltype(slotc)::value;
        constexpr bool FIRST = decltype(firstc)::value;
        constexpr bool TWO = decltype(twoc)::value;
        const int bn = bc == 2 ? 0 : bc + 1;   // next position's buffer
        const int bw = bn == 2 ? 0 : bn + 1;   // buffer of position p+2
        auto steps = [&](int s, int t0) __attribute__((always_inline)) {
            const f32x4(&A)[2][2] = av[s & 1];
#pragma unroll
            for (int t = t0; t < t0 + 4; ++t) {
                if (FIRST && t == 0) {
                    const f32x16 z = {};
                    acc[0][s] = g16_step(A[0][0][0], wc[0], z);
                    if constexpr (TWO) acc[1][s] = g16_step(A[1][0][0], wc[0], z);
                } else {
                    acc[0][s] = g16_step(A[0][t >> 2][t & 3], wc[t], acc[0][s]);
                    if constexpr (TWO) acc[1][s] = g16_step(A[1][t >> 2][t & 3], wc[t], acc[1][s]);
                }
            }
        };
#pragma unroll
        for (int s = 0; s < 4; ++s) {
            if (s < 3)
                read_a(bc, s + 1, av[(s + 1) & 1]);
            else
                read_a(bn, 0, av[0]);
            __builtin_amdgcn_sched_barrier(0);
            steps(s, 0);
            __builtin_amdgcn_sched_barrier(0);
            float wn[8];
            if (s < 3)
                widen_slot(ring[SL][s + 1], s + 1, lastw, wn);
            else
                widen_slot(ring[SL ^ 1][0], 0, lastn, wn);
            load_w(Lw, lrw, s, ring[SL][s]);  // its weights were widened one set ago
            if (s == 2) {
                store_x(bw, lrw, stg);  // position p+2 (its round index is lrw)
                load_x(Lx, lrx, stg);
            }
            g16_pin();
            __builtin_amdgcn_sched_barrier(0);
            steps(s, 4);
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int t = 0; t < 8; ++t) wc[t] = wn[t];
        }
        bc = bn;
        __syncthreads();
    };
    // All R rounds of one job (R >= 3), the first in register slot S0 (round
    // r in slot S0 ^ (r & 1)).  Round r loads the weights of round r+2 and
    // the activations of round r+3 of this job (Lc) while those exist, else
    // the first rounds of the next job (Ln).
    auto job_rounds = [&](auto s0c, auto twoc, const LoadState& Ln) __attribute__((always_inline)) {
        constexpr int S0 = decltype(s0c)::value;
        constexpr int SA = S0 ^ (ODD ? 0 : 1);  // slot of round R-3
        using T = decltype(twoc);
        using F = BoolC2<false>;
        if (R == 3) {
            round(IntC2<S0>{}, BoolC2<true>{}, T{}, Lc, 2, Ln, 0, false, false);
            round(IntC2<S0 ^ 1>{}, F{}, T{}, Ln, 0, Ln, 1, false, true);
            round(IntC2<S0>{}, F{}, T{}, Ln, 1, Ln, 2, true, false);
            return;
        }
        round(IntC2<S0>{}, BoolC2<true>{}, T{}, Lc, 2, Lc, 3, false, false);
        int r = 1;  // rounds 1 .. R-4 read this job only
        for (; r + 2 <= R - 3; r += 2) {
            round(IntC2<S0 ^ 1>{}, F{}, T{}, Lc, r + 2, Lc, r + 3, false, false);
            round(IntC2<S0>{}, F{}, T{}, Lc, r + 3, Lc, r + 4, false, false);
        }
        if (r < R - 3) round(IntC2<S0 ^ 1>{}, F{}, T{}, Lc, r + 2, Lc, r + 3, false, false);
        round(IntC2<SA>{}, F{}, T{}, Lc, R - 1, Ln, 0, false, false);
        round(IntC2<SA ^ 1>{}, F{}, T{}, Ln, 0, Ln, 1, false, true);
        round(IntC2<SA>{}, F{}, T{}, Ln, 1, Ln, 2, true, false);
    };

    int s0 = 0;  // register slot of the compute job's first round
    for (uint32_t ci = 0; ci < my_jobs; ++ci) {
        const G16Job cj = decode(ci);
        // the next job's load state (the last job repeats itself: its loads
        // stay in bounds and are never used)
        const LoadState Ln = ci + 1 < my_jobs ? load_state(decode(ci + 1)) : Lc;
        const bool two = cj.rc > 16;
        // each variant ends with its own finish: no control-flow merge sits
        // between a job's last round and its stores, so the waits before
        // the stores follow that variant's own loads in flight
        if (!ODD || s0 == 0) {
            if (two) {
                job_rounds(IntC2<0>{}, BoolC2<true>{}, Ln);
                finish(cj, BoolC2<true>{});
            } else {
                job_rounds(IntC2<0>{}, BoolC2<false>{}, Ln);
                finish(cj, BoolC2<false>{});
            }
        } else {
            if (two) {
                job_rounds(IntC2<1>{}, BoolC2<true>{}, Ln);
                finish(cj, BoolC2<true>{});
            } else {
                job_rounds(IntC2<1>{}, BoolC2<false>{}, Ln);
                finish(cj, BoolC2<false>{});
            }
        }
        Lc = Ln;
        if (ODD) s0 ^= 1;
    }
}

template <int DT>
auto g16_pick(bool odd, bool tail) {
    return odd ? (tail ? grouped16_kernel<DT, true, true> : grouped16_kernel<DT, true, false>)
               : (tail ? grouped16_kernel<DT, false, true> : grouped16_kernel<DT, false, false>);
}


// A persistent grid: at most one block per compute unit (rounded up to the
// 8 XCDs) and no more blocks than jobs.  The dynamic LDS limit is raised
// once per kernel.
hipError_t g16_launch(const MatmulArgs& a, const MapBuffers& buf, int device_cus, hipStream_t stream) {
    const uint64_t routed = (uint64_t)a.m * a.top_k;
    const uint64_t ntiles = (a.n + kG16BN - 1) / kG16BN;
    const uint64_t job_bound = (routed / kG16BM + a.n_experts + 1) * ntiles;
    const bool tail = a.k % kRoundK != 0;
    const bool odd = ((a.k + kRoundK - 1) / kRoundK) % 2 == 1;
    auto kernel = a.dtype == kDtypeF16 ? g16_pick<kDtypeF16>(odd, tail) : g16_pick<kDtypeBF16>(odd, tail);
    const size_t lds = (size_t)kG16XBufs * kG16XBuf + 4 * (size_t)kG16Ent * sizeof(uint32_t) +
                       (3 * (size_t)a.n_experts + 4) * sizeof(uint32_t);
    // more than the default 64 KB of dynamic LDS: raise the kernel's limit
    // once (a host-side attribute, not a stream operation)
    static std::atomic<uint32_t> raised{0};
    const uint32_t bit = 1u << ((a.dtype == kDtypeF16 ? 4 : 0) + (odd ? 2 : 0) + (tail ? 1 : 0));
    if (!(raised.load(std::memory_order_relaxed) & bit)) {
        const hipError_t err = hipFuncSetAttribute(reinterpret_cast<const void*>(kernel),
                                                   hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (err != hipSuccess) return err;
        raised.fetch_or(bit, std::memory_order_relaxed);
    }
    const uint64_t resident = (uint64_t)(device_cus > 0 ? device_cus : 256);
    uint64_t grid = job_bound < resident ? job_bound : resident;
    grid = (grid + kG16Xcds - 1) / kG16Xcds * kG16Xcds;
    hipLaunchKernelGGL(kernel, dim3((uint32_t)grid), dim3(kG16Threads), lds, stream, a, buf.counts, buf.offsets,
                       buf.rows);
    return launched(EIDM_KERNEL_GROUPED_16X16, (uint32_t)grid, kG16Threads, (uint32_t)lds);
}

}  // namespace
}  // namespace eidm
