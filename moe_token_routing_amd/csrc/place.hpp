// The place step of moe_dispatch (the launch after the tile histograms),
// as a device function of the block index, so that it can run in a kernel
// of its own or beside other work in one launch.
//
// Method: lmdeploy PR #4835, MoE gate v2 notes (stable scatter of the
// routed slots, ranks by flat index, -1 fills).
#pragma once

#include "common.hpp"

namespace moe {
namespace {

constexpr int kDispBlock = 256;
constexpr int kDispWaves = kDispBlock / kWave;
constexpr int kHistBatch = 32;                // tile histograms loaded before they are added
// Rows of four-expert groups in flight per lane in the fused sum (E % 4 ==
// 0): one round of loads at 64 tiles; measured 9.1 -> 8.1 us for the place
// step at 8192 tokens, top-8 of 256, against one expert per thread.
constexpr int kSumBatch = 16;
constexpr int kIdChunks = 16;                 // 64-slot chunks of a wave's quarter held in registers

__device__ __forceinline__ int slot_id(const int32_t* ids, int f, int n, int E) {
    if (f >= n) return -1;
    const int v = ids[f];
    return (v >= 0 && v < E) ? v : -1;
}

// Ranks one 64-slot chunk (lane = slot f within the chunk) among the chunk's
// slots with the same id and places it: equal ids are matched with ballots
// over the id bits, so the rank is the number of earlier slots with that id.
// run[id] holds the next free position of the wave's run of expert id.
__device__ __forceinline__ void place_chunk(int id, int f, int n, int E, int idbits,
                                            int32_t* run, int32_t* __restrict__ perm,
                                            int32_t* __restrict__ dest) {
    const int key = id >= 0 ? id : E;   // ids < E, and E itself marks "no entry"
    uint64_t peers = ~0ull;
    for (int b = 0; b < idbits; ++b) {
        const bool bit = (key >> b) & 1;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
    }
    if (id >= 0) {
        const int rank = __popcll(peers & lanemask_lt());
        const int pos = run[id] + rank;
        perm[pos] = f;
        dest[f] = pos;
        // the last peer lane advances the running position of this id
        if ((peers >> __lane_id()) == 1ull) run[id] = pos + 1;
    } else if (f < n) {
        dest[f] = -1;
    }
}

// How the place step learns the expert totals and its tile's prefix.
enum PlaceMode {
    kPlaceScanned = 0,   // tile_hist holds the prefixes and counts the totals, from scan_kernel
    kPlaceFused = 1,     // tile_hist holds the raw tile histograms; the block sums them itself
    kPlaceSingle = 2     // one tile: its per-wave histograms give the totals (no hist_kernel)
};

// Entries of `off` in the place step's LDS: E + 1, padded to a multiple of
// four so that the arrays after it start 16-byte aligned (E % 4 == 0).
__host__ __device__ constexpr int place_off_len(int E) { return (E + 4) & ~3; }

// Place block `blk` (the tile index); lds: the block's dynamic LDS
// (place_lds_bytes), laid out as off[place_off_len(E)], hist[kDispWaves][E],
// then (fused, single) cnt[E], rel[E]. Block 0 writes the totals to counts
// in the fused and single modes.
template <int MODE>
__device__ __forceinline__ void place_body(
    int blk, int32_t* lds, const int32_t* __restrict__ ids, int n, int E, int tile, int tiles,
    const int32_t* __restrict__ tile_hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ dest) {
    int32_t* off = lds;
    int32_t* hist = lds + place_off_len(E);
    __shared__ int32_t wsum[kDispWaves];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    // The wave's quarter of the tile, in 64-slot chunks. Up to kIdChunks
    // chunks are loaded into registers here, before the tile sums, so their
    // latency overlaps; steps (2) and (4) then read no ids from memory.
    const int base = blk * tile;
    const int quarter = tile / kDispWaves;          // multiple of 64
    const int q0 = base + wave * quarter;
    const int nchunks = quarter / kWave;
    const bool cached = nchunks <= kIdChunks;
    int idr[kIdChunks];
    if (cached) {
#pragma unroll
        for (int c = 0; c < kIdChunks; ++c)
            idr[c] = c < nchunks ? slot_id(ids, q0 + c * kWave + lane, n, E) : -1;
    }
    const int32_t* cnt = counts;
    const int32_t* rel = tile_hist + static_cast<size_t>(blk) * E;
    int32_t* my = hist + wave * E;
    if (MODE == kPlaceSingle) {
        // step (2) first: the per-wave histograms, then the totals from them
        for (int e = tid; e < kDispWaves * E; e += kDispBlock) hist[e] = 0;
        __syncthreads();
        if (cached) {
#pragma unroll
            for (int c = 0; c < kIdChunks; ++c)
                if (idr[c] >= 0) atomicAdd(&my[idr[c]], 1);
        } else {
            for (int i = lane; i < quarter; i += kWave) {
                const int id = slot_id(ids, q0 + i, n, E);
                if (id >= 0) atomicAdd(&my[id], 1);
            }
        }
        __syncthreads();
        int32_t* cnt_l = hist + kDispWaves * E;
        int32_t* rel_l = cnt_l + E;
        for (int e = tid; e < E; e += kDispBlock) {
            int total = 0;
#pragma unroll
            for (int w = 0; w < kDispWaves; ++w) total += hist[w * E + e];
            cnt_l[e] = total;
            rel_l[e] = 0;
            counts[e] = total;
        }
        __syncthreads();
        cnt = cnt_l;
        rel = rel_l;
    }
    if (MODE == kPlaceFused && (E & 3) == 0) {
        // Wave w sums tiles [w per, (w + 1) per) for groups of four experts
        // (16-byte loads, a batch of kSumBatch rows in flight per lane);
        // the partial totals meet in LDS. The exclusive prefix over tiles
        // before this block's own is the totals of the waves whose tiles all
        // lie before it plus a partial sum kept by the one wave holding it.
        int32_t* cnt_l = hist + kDispWaves * E;
        int32_t* rel_l = cnt_l + E;
        const int b = blk;
        const int per = (tiles + kDispWaves - 1) / kDispWaves;
        const int t0 = wave * per, t1 = min(tiles, t0 + per);
        const int bw = b / per;
        const int groups = E >> 2;
        for (int g = lane; g < groups; g += kWave) {
            int4 tot = make_int4(0, 0, 0, 0), bef = make_int4(0, 0, 0, 0);
#pragma unroll 1
            for (int ta = t0; ta < t1; ta += kSumBatch) {
                int4 v[kSumBatch];
#pragma unroll
                for (int u = 0; u < kSumBatch; ++u)
                    v[u] = ta + u < t1 ? reinterpret_cast<const int4*>(tile_hist + static_cast<size_t>(ta + u) * E)[g]
                                       : make_int4(0, 0, 0, 0);
#pragma unroll
                for (int u = 0; u < kSumBatch; ++u) {
                    tot.x += v[u].x; tot.y += v[u].y; tot.z += v[u].z; tot.w += v[u].w;
                    if (ta + u < b) { bef.x += v[u].x; bef.y += v[u].y; bef.z += v[u].z; bef.w += v[u].w; }
                }
            }
            reinterpret_cast<int4*>(hist + wave * E)[g] = tot;
            if (wave == bw) reinterpret_cast<int4*>(rel_l)[g] = bef;
        }
        __syncthreads();
        for (int e = tid; e < E; e += kDispBlock) {
            int total = 0, before = rel_l[e];
#pragma unroll
            for (int w = 0; w < kDispWaves; ++w) {
                const int c = hist[w * E + e];
                total += c;
                if (w < bw) before += c;
            }
            cnt_l[e] = total;
            rel_l[e] = before;
            if (b == 0) counts[e] = total;
        }
        __syncthreads();
        cnt = cnt_l;
        rel = rel_l;
    } else if (MODE == kPlaceFused) {
        int32_t* cnt_l = hist + kDispWaves * E;
        int32_t* rel_l = cnt_l + E;
        for (int e = tid; e < E; e += kDispBlock) {
            int before = 0, total = 0;
#pragma unroll 1
            for (int t0 = 0; t0 < tiles; t0 += kHistBatch) {
                int v[kHistBatch];
#pragma unroll
                for (int u = 0; u < kHistBatch; ++u)
                    v[u] = t0 + u < tiles ? tile_hist[static_cast<size_t>(t0 + u) * E + e] : 0;
#pragma unroll
                for (int u = 0; u < kHistBatch; ++u) {
                    total += v[u];
                    if (t0 + u < blk) before += v[u];
                }
            }
            cnt_l[e] = total;
            rel_l[e] = before;
            if (blk == 0) counts[e] = total;
        }
        __syncthreads();
        cnt = cnt_l;
        rel = rel_l;
    }

    // (1) offsets = exclusive scan of counts: contiguous chunk per thread.
    const int chunk = (E + kDispBlock - 1) / kDispBlock;
    const int c0 = min(E, tid * chunk), c1 = min(E, c0 + chunk);
    int local = 0;
    for (int e = c0; e < c1; ++e) local += cnt[e];
    int incl = local;   // inclusive scan over the block, in thread order
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    if (MODE != kPlaceSingle)
        for (int e = tid; e < kDispWaves * E; e += kDispBlock) hist[e] = 0;
    __syncthreads();
    int before = 0;
    for (int w = 0; w < wave; ++w) before += wsum[w];
    int run = before + incl - local;
    for (int e = c0; e < c1; ++e) {
        off[e] = run;
        run += cnt[e];
    }
    if (tid == kDispBlock - 1) off[E] = before + incl;
    __syncthreads();
    const int total = off[E];
    if (blk == 0)
        for (int e = tid; e <= E; e += kDispBlock) offsets[e] = off[e];

    // (2) per-wave histograms of the tile's quarters (done above for one tile).
    if (MODE != kPlaceSingle) {
        if (cached) {
#pragma unroll
            for (int c = 0; c < kIdChunks; ++c)
                if (idr[c] >= 0) atomicAdd(&my[idr[c]], 1);
        } else {
            for (int i = lane; i < quarter; i += kWave) {
                const int id = slot_id(ids, q0 + i, n, E);
                if (id >= 0) atomicAdd(&my[id], 1);
            }
        }
        __syncthreads();
    }
    // (3) starting position of each wave's run of each expert.
    for (int e = tid; e < E; e += kDispBlock) {
        int p = off[e] + rel[e];
#pragma unroll
        for (int w = 0; w < kDispWaves; ++w) {
            const int c = hist[w * E + e];
            hist[w * E + e] = p;
            p += c;
        }
    }
    __syncthreads();
    // (4) rank and place, 64 slots at a time, in slot order within each wave.
    const int idbits = 32 - __clz(E);
    if (cached) {
#pragma unroll
        for (int c = 0; c < kIdChunks; ++c)
            if (c < nchunks) place_chunk(idr[c], q0 + c * kWave + lane, n, E, idbits, my, perm, dest);
    } else {
        for (int i0 = 0; i0 < quarter; i0 += kWave) {
            const int f = q0 + i0 + lane;
            place_chunk(slot_id(ids, f, n, E), f, n, E, idbits, my, perm, dest);
        }
    }
    // (5) positions past the last valid entry hold -1; each tile clears its own range.
    for (int p = base + tid; p < base + tile && p < n; p += kDispBlock)
        if (p >= total) perm[p] = -1;
}

// Bytes of dynamic LDS of the place step in mode `mode`.
inline size_t place_lds_bytes(int mode, int E) {
    const size_t base =
        sizeof(int32_t) * (static_cast<size_t>(place_off_len(E)) + static_cast<size_t>(kDispWaves) * E);
    return mode == kPlaceScanned ? base : base + sizeof(int32_t) * 2 * E;
}

}  // namespace
}  // namespace moe
