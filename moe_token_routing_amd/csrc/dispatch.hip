// moe_dispatch: expert histogram, exclusive prefix scan and stable permutation
// of the routed slots.
//
// Method: lmdeploy PR #4835 ("Intern-S2-Mobius meta-MoE support, MoE gate v2,
// CP attention fixes"), MoE gate v2 notes: per-tile shared-memory expert
// histograms, a hierarchical multi-block scan over the tiles for large E, the
// required validity mask (invalid slots get no entry) and the slot-to-position
// map cleared to -1.
//
// Three launches, all deterministic:
//   1. hist   one block per tile of slots: LDS histogram of the tile's valid
//             ids, written as tile_counts[tile][E]. (moe_route_dispatch
//             skips it: its selection counts the picks into the same
//             histograms with integer atomics.)
//   2. scan   blocks over 64-expert columns: for each expert, the exclusive
//             prefix of its count over the tiles (in place) and its total.
//   3. place  one block per tile: offsets from the totals (block-wide scan),
//             per-wave LDS histograms of the tile's four quarters, then each
//             wave ranks its 64-slot chunks in slot order. Equal ids within a
//             chunk are matched with ballots over the id bits, so the rank
//             of a slot is the number of earlier slots with its id: the order
//             within an expert is ascending slot index.
// When the tile histograms are small (tiles^2 * E at most kFuseLimit: up to
// tens of thousands of slots over a few hundred experts), step 2 is folded
// into step 3: each place block sums the histograms itself -- its own
// exclusive prefix over the tiles and every expert's total -- which saves a
// launch (the four waves each sum a quarter of the tiles, 16-byte loads of
// four experts at a time, and meet in LDS). With one tile (up to 1024 slots)
// step 1 goes too: the place block's per-wave histograms are the only ones,
// and their sums are the totals.
#include <atomic>
#include <cmath>

#include "dispatch.hpp"
#include "launch.hpp"

namespace moe {
namespace {

constexpr int kDispBlock = 256;
constexpr int kDispWaves = kDispBlock / kWave;
constexpr int kMaxTiles = 256;
// tiles * tiles * E read by the fused place step: 64 tiles of 256 experts
// (8192 tokens, top-8) stay fused (13 us against 16 us unfused); 32 tiles
// of 2560 experts take the separate scan (19 us against 28 us fused)
constexpr long long kFuseLimit = 1ll << 21;
constexpr int kHistBatch = 32;                // tile histograms loaded before they are added
// Rows of four-expert groups in flight per lane in the fused sum (E % 4 ==
// 0): one round of loads at 64 tiles; measured 9.1 -> 8.1 us for the place
// step at 8192 tokens, top-8 of 256, against one expert per thread.
constexpr int kSumBatch = 16;
constexpr int kIdBatch = 16;                  // ids per thread loaded before they are counted
constexpr int kIdChunks = 16;                 // 64-slot chunks of a wave's quarter held in registers

struct TilePlan {
    int n;        // slots
    int tiles;
    int tile;     // slots per tile, a multiple of kDispBlock
};

inline TilePlan plan_tiles(long long n) {
    TilePlan p;
    p.n = static_cast<int>(n);
    long long tiles = (n + 1023) / 1024;
    if (tiles > kMaxTiles) tiles = kMaxTiles;
    if (tiles < 1) tiles = 1;
    long long per = (n + tiles - 1) / tiles;
    per = (per + kDispBlock - 1) / kDispBlock * kDispBlock;
    if (per < kDispBlock) per = kDispBlock;
    p.tile = static_cast<int>(per);
    p.tiles = static_cast<int>((n + per - 1) / per);
    if (p.tiles < 1) p.tiles = 1;
    return p;
}

__device__ __forceinline__ int slot_id(const int32_t* ids, int f, int n, int E) {
    if (f >= n) return -1;
    const int v = ids[f];
    return (v >= 0 && v < E) ? v : -1;
}

__global__ __launch_bounds__(kDispBlock) void hist_kernel(const int32_t* __restrict__ ids, int n,
                                                          int E, int tile,
                                                          int32_t* __restrict__ tile_counts) {
    extern __shared__ int32_t lds[];
    for (int e = threadIdx.x; e < E; e += kDispBlock) lds[e] = 0;
    __syncthreads();
    const int base = blockIdx.x * tile;
    // kIdBatch ids per thread are loaded before any is counted, so a tile of
    // up to kIdBatch * kDispBlock slots costs one memory round trip
    for (int i0 = threadIdx.x; i0 < tile; i0 += kIdBatch * kDispBlock) {
        int id[kIdBatch];
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u) {
            const int i = i0 + u * kDispBlock;
            id[u] = i < tile ? slot_id(ids, base + i, n, E) : -1;
        }
#pragma unroll
        for (int u = 0; u < kIdBatch; ++u)
            if (id[u] >= 0) atomicAdd(&lds[id[u]], 1);
    }
    __syncthreads();
    int32_t* row = tile_counts + static_cast<size_t>(blockIdx.x) * E;
    for (int e = threadIdx.x; e < E; e += kDispBlock) row[e] = lds[e];
}

// Block: 64 experts (lane) x 4 segments of tiles (wave).
__global__ __launch_bounds__(kDispBlock) void scan_kernel(int32_t* __restrict__ tile_counts,
                                                          int tiles, int E,
                                                          int32_t* __restrict__ counts) {
    __shared__ int32_t part[kDispWaves][kWave];
    const int lane = __lane_id();
    const int seg = threadIdx.x / kWave;
    const int e = blockIdx.x * kWave + lane;
    const int per = (tiles + kDispWaves - 1) / kDispWaves;
    const int t0 = seg * per;
    const int t1 = min(tiles, t0 + per);
    int sum = 0;
    if (e < E) {
#pragma unroll 8
        for (int t = t0; t < t1; ++t) sum += tile_counts[static_cast<size_t>(t) * E + e];
    }
    part[seg][lane] = sum;
    __syncthreads();
    int run = 0;
    for (int s = 0; s < seg; ++s) run += part[s][lane];
    if (e < E) {
        if (seg == kDispWaves - 1) counts[e] = run + sum;
        for (int t = t0; t < t1; ++t) {
            int32_t* p = tile_counts + static_cast<size_t>(t) * E + e;
            const int c = *p;
            *p = run;
            run += c;
        }
    }
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

// LDS layout: off[place_off_len(E)], hist[kDispWaves][E], then (fused,
// single) cnt[E], rel[E]. Block 0 writes the totals to counts in the fused
// and single modes.
template <int MODE>
__global__ __launch_bounds__(kDispBlock) void place_kernel(
    const int32_t* __restrict__ ids, int n, int E, int tile, int tiles,
    const int32_t* __restrict__ tile_hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ dest) {
    extern __shared__ __attribute__((aligned(16))) int32_t lds[];
    int32_t* off = lds;
    int32_t* hist = lds + place_off_len(E);
    __shared__ int32_t wsum[kDispWaves];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    // The wave's quarter of the tile, in 64-slot chunks. Up to kIdChunks
    // chunks are loaded into registers here, before the tile sums, so their
    // latency overlaps; steps (2) and (4) then read no ids from memory.
    const int base = blockIdx.x * tile;
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
    const int32_t* rel = tile_hist + static_cast<size_t>(blockIdx.x) * E;
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
        const int b = blockIdx.x;
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
                    if (t0 + u < static_cast<int>(blockIdx.x)) before += v[u];
                }
            }
            cnt_l[e] = total;
            rel_l[e] = before;
            if (blockIdx.x == 0) counts[e] = total;
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
    if (blockIdx.x == 0)
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

__global__ __launch_bounds__(kDispBlock) void zero_kernel(int32_t* __restrict__ counts,
                                                          int32_t* __restrict__ offsets, int E) {
    for (int e = threadIdx.x; e <= E; e += kDispBlock) {
        if (e < E) counts[e] = 0;
        offsets[e] = 0;
    }
}

// Clears n int32 (the tile histograms the selection then counts into): a
// kernel, not a memset node, so that a captured graph replays it faithfully.
__global__ __launch_bounds__(kDispBlock) void clear_kernel(int32_t* __restrict__ p, long long n) {
    for (long long i = blockIdx.x * static_cast<long long>(kDispBlock) + threadIdx.x; i < n;
         i += static_cast<long long>(gridDim.x) * kDispBlock)
        p[i] = 0;
}

}  // namespace

DispatchTiles dispatch_tiles(long long n) {
    const TilePlan p = plan_tiles(n);
    return DispatchTiles{p.tiles, p.tile};
}

int run_dispatch_empty(int32_t* counts, int32_t* offsets, int E, void* stream) {
    return launch(zero_kernel, dim3(1), dim3(kDispBlock), 0, stream, counts, offsets, E);
}

int run_clear(int32_t* p, long long n, void* stream) {
    if (n <= 0) return MOE_OK;
    const long long blocks = (n + kDispBlock - 1) / kDispBlock;
    return launch(clear_kernel, dim3(static_cast<unsigned>(blocks < 1024 ? blocks : 1024)), dim3(kDispBlock), 0,
                  stream, p, n);
}

// The launches after the tile histograms exist (tile_counts[tile][E], raw
// counts of the valid slots of each tile; with one tile nothing is read:
// its place block counts the tile itself).
int run_place(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
              int32_t* dest, int32_t* tile_counts, void* stream) {
    const TilePlan p = plan_tiles(n);
    const size_t lds = sizeof(int32_t) * (static_cast<size_t>(place_off_len(E)) + static_cast<size_t>(kDispWaves) * E);
    if (p.tiles == 1)
        return launch(place_kernel<kPlaceSingle>, dim3(1), dim3(kDispBlock), lds + sizeof(int32_t) * 2 * E,
                      stream, topk_ids, p.n, E, p.tile, p.tiles, static_cast<const int32_t*>(tile_counts),
                      counts, offsets, perm, dest);
    if (static_cast<long long>(p.tiles) * p.tiles * E <= kFuseLimit)
        return launch(place_kernel<kPlaceFused>, dim3(p.tiles), dim3(kDispBlock), lds + sizeof(int32_t) * 2 * E,
                      stream, topk_ids, p.n, E, p.tile, p.tiles, static_cast<const int32_t*>(tile_counts),
                      counts, offsets, perm, dest);
    const int rc = launch(scan_kernel, dim3(ceil_div(E, kWave)), dim3(kDispBlock), 0, stream, tile_counts,
                          p.tiles, E, counts);
    if (rc) return rc;
    return launch(place_kernel<kPlaceScanned>, dim3(p.tiles), dim3(kDispBlock), lds, stream, topk_ids, p.n, E,
                  p.tile, p.tiles, static_cast<const int32_t*>(tile_counts), counts, offsets, perm, dest);
}

// The launches of one dispatch, given the tile histogram scratch
// (moe_dispatch_workspace_bytes(T, k, E) bytes; every entry a launch reads
// is written earlier in the same call, so nothing needs clearing).
int run_dispatch(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
                 int32_t* dest, int32_t* tile_counts, void* stream) {
    const TilePlan p = plan_tiles(n);
    if (p.tiles > 1) {
        const int rc = launch(hist_kernel, dim3(p.tiles), dim3(kDispBlock), sizeof(int32_t) * E, stream,
                              topk_ids, p.n, E, p.tile, tile_counts);
        if (rc) return rc;
    }
    return run_place(topk_ids, n, E, counts, offsets, perm, dest, tile_counts, stream);
}

int check_dispatch(const int32_t* topk_ids, int T, int k, int E, const int32_t* counts, const int32_t* offsets,
                   const int32_t* perm, const int32_t* dest) {
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_BAD_SHAPE;
    const long long n = static_cast<long long>(T) * k;
    if (n >= (1ll << 31)) return MOE_ERR_BAD_SHAPE;
    if (!counts || !offsets) return MOE_ERR_NULL_ARG;
    if (n > 0 && (!topk_ids || !perm || !dest)) return MOE_ERR_NULL_ARG;
    if (!all_aligned16(topk_ids, counts, offsets, perm, dest)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

// Scratch of the allocation-free dispatch: the per-tile expert histograms,
// at most kMaxTiles x MOE_MAX_EXPERTS int32 (4 MiB), which every supported
// shape fits. One copy per GPU the library runs on, held until the process
// ends. Host code never passes this name to a kernel (on the host it is only
// a handle); it uses the device address hipGetSymbolAddress returns.
static __device__ __align__(256) int32_t scratch[kMaxTiles * MOE_MAX_EXPERTS];

namespace {

constexpr int kMaxDevices = 64;

// Device address of `scratch` on the current device, looked up once per
// device (threads racing on the first lookup store the same address).
int32_t* scratch_address(int* status) {
    static std::atomic<int32_t*> cached[kMaxDevices];
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        *status = MOE_ERR_HIP;
        return nullptr;
    }
    int32_t* ptr = cached[dev].load(std::memory_order_acquire);
    if (!ptr) {
        void* addr = nullptr;
        if (hipGetSymbolAddress(&addr, HIP_SYMBOL(scratch)) != hipSuccess || !addr) {
            *status = MOE_ERR_HIP;
            return nullptr;
        }
        ptr = static_cast<int32_t*>(addr);
        cached[dev].store(ptr, std::memory_order_release);
    }
    *status = MOE_OK;
    return ptr;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_dispatch_workspace_bytes(int T, int k, int E) {
    using namespace moe;
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    const long long n = static_cast<long long>(T) * k;
    if (n == 0) return 0;
    const TilePlan p = plan_tiles(n);
    const size_t bytes = static_cast<size_t>(p.tiles) * E * sizeof(int32_t);
    return (bytes + 255) / 256 * 256;
}

extern "C" int moe_dispatch(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                            int32_t* offsets, int32_t* perm, int32_t* dest, void* workspace,
                            size_t workspace_bytes, void* stream) {
    using namespace moe;
    const int rc = check_dispatch(topk_ids, T, k, E, counts, offsets, perm, dest);
    if (rc) return rc;
    const long long n = static_cast<long long>(T) * k;
    if (n == 0)   // no slots: counts and offsets are all zero (a kernel, not a memset node)
        return run_dispatch_empty(counts, offsets, E, stream);
    const size_t need = moe_dispatch_workspace_bytes(T, k, E);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    return run_dispatch(topk_ids, n, E, counts, offsets, perm, dest, static_cast<int32_t*>(workspace), stream);
}

extern "C" int moe_dispatch_noalloc(const int32_t* topk_ids, int T, int k, int E, int32_t* counts,
                                    int32_t* offsets, int32_t* perm, int32_t* dest, void* stream) {
    using namespace moe;
    const int rc = check_dispatch(topk_ids, T, k, E, counts, offsets, perm, dest);
    if (rc) return rc;
    const long long n = static_cast<long long>(T) * k;
    if (n == 0)
        return run_dispatch_empty(counts, offsets, E, stream);
    if (moe_dispatch_workspace_bytes(T, k, E) > sizeof(scratch)) return MOE_ERR_WORKSPACE;
    int status = MOE_OK;
    int32_t* tile_counts = scratch_address(&status);
    if (status) return status;
    return run_dispatch(topk_ids, n, E, counts, offsets, perm, dest, tile_counts, stream);
}
