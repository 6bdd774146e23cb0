// map_keyed.hpp -- the one-launch form of the id -> row map, as a block
// body: block e of a launch of n_experts + 1 blocks of 1024 threads builds
// key e's entries.  Used by the map kernel (map.hip) and by the split-16
// route's launch that also splits the activations (matmul_split16.hip).
//
// mlx-native 0.13.0, src/ops/dense_matmul_id_auto.rs, fn expected_dispatches:
// the grouped route's map pass builds per-expert row lists.  Key of routed
// row r: min(ids[r], n_experts) (the last bucket gathers ids that name no
// expert); the rows of each key in ascending order (a stable counting sort).
#pragma once

#include "eidm_device.hpp"
#include "eidm_internal.hpp"

namespace eidm {

__device__ __forceinline__ uint32_t map_key_of(uint32_t id, uint32_t n_experts) {
    return id < n_experts ? id : n_experts;
}

__device__ __forceinline__ uint64_t map_lanes_below(int lane) {
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

// One block per key e (1024 threads = 16 wavefronts).  Wavefront w owns the
// contiguous rows [w*span, (w+1)*span), span a multiple of 64, in at most
// kMapKeyedChunks chunks of 64; so (wavefront, chunk, lane) order is row
// order and a running count per wavefront plus a prefix over the
// wavefronts places every row.
constexpr int kMapKeyedWaves = 16;
constexpr int kMapKeyedChunks = 16;
constexpr uint32_t kMapKeyedMaxRows = 64u * kMapKeyedWaves * kMapKeyedChunks;  // 16384

// key e: an expert, or n_experts for ids naming none; the calling block has
// 64 * kMapKeyedWaves threads
__device__ __forceinline__ void map_keyed_block(uint32_t e, const uint32_t* __restrict__ ids, uint32_t routed_rows,
                                                uint32_t n_experts, uint32_t span, uint32_t* __restrict__ counts,
                                                uint32_t* __restrict__ offsets, uint32_t* __restrict__ rows) {
    __shared__ uint32_t lt_s[kMapKeyedWaves], eq_s[kMapKeyedWaves];
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const uint32_t first = (uint32_t)wave * span + (uint32_t)lane;
    const int chunks = (int)(span >> 6);
    // every id of this wavefront's rows first, then the two counts.  The
    // loads are unconditional (rows past the end re-read the last id, and
    // routed_rows >= 1: zero dimensions are rejected on the host), so all
    // of them are in flight together; a load under a branch would be waited
    // for before the next one is issued.
    uint32_t raw[kMapKeyedChunks], key[kMapKeyedChunks];
#pragma unroll
    for (int c = 0; c < kMapKeyedChunks; ++c) raw[c] = ids[min(first + 64u * (uint32_t)c, routed_rows - 1)];
#pragma unroll
    for (int c = 0; c < kMapKeyedChunks; ++c) {
        const uint32_t r = first + 64u * (uint32_t)c;
        key[c] = c < chunks && r < routed_rows ? map_key_of(raw[c], n_experts) : 0xffffffffu;
    }
    uint32_t lt = 0, eq = 0;
#pragma unroll
    for (int c = 0; c < kMapKeyedChunks; ++c) {
        lt += (uint32_t)__popcll(__ballot(key[c] < e));
        eq += (uint32_t)__popcll(__ballot(key[c] == e));
    }
    if (lane == 0) {
        lt_s[wave] = lt;
        eq_s[wave] = eq;
    }
    __syncthreads();
    uint32_t offset = 0, count = 0, before = 0;
#pragma unroll
    for (int w = 0; w < kMapKeyedWaves; ++w) {
        offset += lt_s[w];
        count += eq_s[w];
        if (w < wave) before += eq_s[w];
    }
    if (threadIdx.x == 0) {
        counts[e] = count;
        offsets[e] = offset;
        if (e == 0) offsets[n_experts + 1] = routed_rows;
    }
    uint32_t pos = offset + before;
    const uint64_t below = map_lanes_below(lane);
#pragma unroll
    for (int c = 0; c < kMapKeyedChunks; ++c) {
        const uint64_t m = __ballot(key[c] == e);
        if (key[c] == e) rows[pos + (uint32_t)__popcll(m & below)] = first + 64u * (uint32_t)c;
        pos += (uint32_t)__popcll(m);
    }
}

// the one-launch form reads all routed_rows ids in each of n_experts+1
// blocks: kept to small maps with at most 2^24 id reads in total
inline bool map_keyed_fits(uint32_t routed_rows, uint32_t n_experts) {
    return routed_rows <= kMapKeyedMaxRows && (uint64_t)(n_experts + 1) * routed_rows <= (1ull << 24);
}

// rows per wavefront of the one-launch form: a multiple of 64, at most
// 64 * kMapKeyedChunks
inline uint32_t map_keyed_span(uint32_t routed_rows) {
    const uint32_t per_wave = (routed_rows + kMapKeyedWaves - 1) / kMapKeyedWaves;
    return (per_wave + 63) / 64 * 64;
}

}  // namespace eidm
