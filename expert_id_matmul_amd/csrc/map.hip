// map.hip -- id -> row map for the grouped form: a stable counting sort of
// the routed rows by expert id.
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs, fn expected_dispatches:
// the grouped route runs a map pass over the ids that builds per-expert row
// lists before the grouped tiles; DenseMatmulIdScratch::new sizes its scratch
// by (n_experts, m).
//
// Key of routed row r: min(ids[r], n_experts) (the last bucket gathers ids
// that name no expert).  Two passes over blocks of 64*W rows (W wavefronts,
// as many as the per-wave count tables fit in 64 KB of LDS, at most 16):
//   hist:    per block, rows per key (wave-aggregated LDS atomics);
//   scatter: per block, global position of each row = rows of smaller keys
//            + rows of the same key in earlier blocks + rows of the same key
//            earlier in this block.  The last term is exact and ordered: it
//            is built from each wave's same-key lane masks and a prefix over
//            the block's waves, so the result is deterministic.
// Small maps (up to kMapKeyedMaxRows routed rows, with the ids read per
// block bounded) take one launch instead: block e reads every id and
// counts the rows with key < e (its offset) and key == e (its count) with
// two ballots per 64 ids, then writes its own rows in ascending order.  No
// block waits for another, and the map is the same stable sort (the block
// body is in map_keyed.hpp).
#include "eidm_device.hpp"
#include "eidm_internal.hpp"
#include "map_keyed.hpp"

namespace eidm {
namespace {

constexpr int kMaxMapWaves = 16;

// Lanes of this wavefront whose key equals this lane's key (active lanes only).
__device__ __forceinline__ uint64_t same_key_lanes(uint32_t key, int nbits, bool active) {
    uint64_t mask = __ballot(active);
    for (int bit = 0; bit < nbits; ++bit) {
        const bool set = (key >> bit) & 1u;
        const uint64_t ones = __ballot(active && set);
        mask &= set ? ones : ~ones;
    }
    return mask;
}

// Exclusive scan of a[0..count) in LDS by the whole block; returns the
// total.  `wave_tot` is one word of LDS per wavefront.
__device__ uint32_t block_exclusive_scan(uint32_t* a, uint32_t count, uint32_t* wave_tot) {
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
    const int waves = blockDim.x >> 6;
    const uint32_t per = (count + blockDim.x - 1) / blockDim.x;
    const uint32_t begin = min(count, (uint32_t)tid * per);
    const uint32_t end = min(count, begin + per);
    uint32_t s = 0;
    for (uint32_t i = begin; i < end; ++i) s += a[i];
    uint32_t inc = s;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
        const uint32_t o = __shfl_up(inc, d);
        if (lane >= d) inc += o;
    }
    if (lane == 63) wave_tot[wave] = inc;
    __syncthreads();
    uint32_t before = 0, total = 0;
    for (int w = 0; w < waves; ++w) {
        if (w < wave) before += wave_tot[w];
        total += wave_tot[w];
    }
    uint32_t run = before + inc - s;
    for (uint32_t i = begin; i < end; ++i) {
        const uint32_t v = a[i];
        a[i] = run;
        run += v;
    }
    __syncthreads();
    return total;
}

__global__ __launch_bounds__(64 * kMaxMapWaves) void map_hist_kernel(const uint32_t* __restrict__ ids,
                                                             uint32_t routed_rows,
                                                             uint32_t n_experts, int nbits,
                                                             uint32_t* __restrict__ hist) {
    extern __shared__ uint32_t cnt[];  // n_experts + 1
    const uint32_t buckets = n_experts + 1;
    for (uint32_t i = threadIdx.x; i < buckets; i += blockDim.x) cnt[i] = 0;
    __syncthreads();
    const int lane = threadIdx.x & 63;
    const uint32_t r = blockIdx.x * blockDim.x + threadIdx.x;
    const bool active = r < routed_rows;
    const uint32_t key = active ? map_key_of(ids[r], n_experts) : 0;
    const uint64_t same = same_key_lanes(key, nbits, active);
    if (active && (same & map_lanes_below(lane)) == 0) atomicAdd(&cnt[key], (uint32_t)__popcll(same));
    __syncthreads();
    uint32_t* out = hist + (size_t)blockIdx.x * buckets;
    for (uint32_t i = threadIdx.x; i < buckets; i += blockDim.x) out[i] = cnt[i];
}

__global__ __launch_bounds__(64 * kMaxMapWaves) void map_scatter_kernel(
    const uint32_t* __restrict__ ids, uint32_t routed_rows, uint32_t n_experts, int nbits,
    uint32_t nblocks, const uint32_t* __restrict__ hist, uint32_t* __restrict__ counts,
    uint32_t* __restrict__ offsets, uint32_t* __restrict__ rows) {
    extern __shared__ uint32_t lds[];
    const uint32_t buckets = n_experts + 1;
    uint32_t* base = lds;                       // [buckets]
    uint32_t* earlier = base + buckets;         // [buckets]
    const int waves = blockDim.x >> 6;
    uint32_t* wcnt = earlier + buckets;         // [waves][buckets]
    uint32_t* wave_tot = wcnt + waves * buckets;  // [waves]
    const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;

    for (uint32_t b = tid; b < buckets; b += blockDim.x) {
        uint32_t tot = 0, pre = 0;
#pragma unroll 8
        for (uint32_t c = 0; c < nblocks; ++c) {
            const uint32_t h = hist[(size_t)c * buckets + b];
            tot += h;
            if (c < blockIdx.x) pre += h;
        }
        base[b] = tot;
        earlier[b] = pre;
        if (blockIdx.x == 0) counts[b] = tot;
    }
    for (uint32_t i = tid; i < waves * buckets; i += blockDim.x) wcnt[i] = 0;
    __syncthreads();
    block_exclusive_scan(base, buckets, wave_tot);
    for (uint32_t b = tid; b < buckets; b += blockDim.x) {
        if (blockIdx.x == 0) offsets[b] = base[b];
        base[b] += earlier[b];
    }
    if (blockIdx.x == 0 && tid == 0) offsets[buckets] = routed_rows;

    const uint32_t r = blockIdx.x * blockDim.x + tid;
    const bool active = r < routed_rows;
    const uint32_t key = active ? map_key_of(ids[r], n_experts) : 0;
    const uint64_t same = same_key_lanes(key, nbits, active);
    const uint32_t rank = (uint32_t)__popcll(same & map_lanes_below(lane));
    if (active && rank == 0) wcnt[wave * buckets + key] = (uint32_t)__popcll(same);
    __syncthreads();
    for (uint32_t b = tid; b < buckets; b += blockDim.x) {
        uint32_t run = 0;
        for (int w = 0; w < waves; ++w) {
            const uint32_t v = wcnt[w * buckets + b];
            wcnt[w * buckets + b] = run;
            run += v;
        }
    }
    __syncthreads();
    if (active) rows[base[key] + wcnt[wave * buckets + key] + rank] = r;
}

__global__ __launch_bounds__(64 * kMapKeyedWaves) void map_keyed_kernel(
    const uint32_t* __restrict__ ids, uint32_t routed_rows, uint32_t n_experts, uint32_t span,
    uint32_t* __restrict__ counts, uint32_t* __restrict__ offsets, uint32_t* __restrict__ rows) {
    map_keyed_block(blockIdx.x, ids, routed_rows, n_experts, span, counts, offsets, rows);
}

int key_bits(uint32_t n_experts) {
    int bits = 0;
    while ((1u << bits) <= n_experts) ++bits;  // keys 0..n_experts
    return bits;
}

}  // namespace

uint32_t map_waves(uint32_t n_experts) {
    // (2 + W) count tables of n_experts+1 words plus W words within 64 KB
    const uint32_t fit = 16384u / (n_experts + 2) - 2;
    uint32_t w = 1;
    while (w * 2 <= fit && w * 2 <= (uint32_t)kMaxMapWaves) w *= 2;
    return w;
}

uint32_t map_blocks(uint64_t routed_rows, uint32_t n_experts) {
    const uint32_t chunk = 64 * map_waves(n_experts);
    return (uint32_t)((routed_rows + chunk - 1) / chunk);
}

uint64_t map_hist_elements(uint64_t routed_rows, uint32_t n_experts) {
    return (uint64_t)map_blocks(routed_rows, n_experts) * (n_experts + 1);
}

hipError_t launch_map(const uint32_t* ids, uint32_t routed_rows, uint32_t n_experts,
                      const MapBuffers& buf, hipStream_t stream) {
    if (map_keyed_fits(routed_rows, n_experts)) {
        const uint32_t span = map_keyed_span(routed_rows);
        hipLaunchKernelGGL(map_keyed_kernel, dim3(n_experts + 1), dim3(64 * kMapKeyedWaves), 0, stream, ids,
                           routed_rows, n_experts, span, buf.counts, buf.offsets, buf.rows);
        return launched(EIDM_KERNEL_MAP_ONE_PASS, n_experts + 1, 64 * kMapKeyedWaves, 0);
    }
    const uint32_t waves = map_waves(n_experts);
    const uint32_t blocks = map_blocks(routed_rows, n_experts);
    const uint32_t buckets = n_experts + 1;
    const int nbits = key_bits(n_experts);
    hipLaunchKernelGGL(map_hist_kernel, dim3(blocks), dim3(64 * waves), buckets * sizeof(uint32_t),
                       stream, ids, routed_rows, n_experts, nbits, buf.hist);
    hipError_t err = launched(EIDM_KERNEL_MAP_HISTOGRAM, blocks, 64 * waves, buckets * sizeof(uint32_t));
    if (err != hipSuccess) return err;
    const size_t lds = ((2 + waves) * (size_t)buckets + waves) * sizeof(uint32_t);
    hipLaunchKernelGGL(map_scatter_kernel, dim3(blocks), dim3(64 * waves), lds, stream, ids,
                       routed_rows, n_experts, nbits, blocks, buf.hist, buf.counts, buf.offsets,
                       buf.rows);
    return launched(EIDM_KERNEL_MAP_SCATTER, blocks, 64 * waves, (uint32_t)lds);
}

}  // namespace eidm
