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
#include "place.hpp"

namespace moe {
namespace {

constexpr int kMaxTiles = 256;
// tiles * tiles * E read by the fused place step: 64 tiles of 256 experts
// (8192 tokens, top-8) stay fused (13 us against 16 us unfused); 32 tiles
// of 2560 experts take the separate scan (19 us against 28 us fused)
constexpr long long kFuseLimit = 1ll << 21;
constexpr int kIdBatch = 16;                  // ids per thread loaded before they are counted

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

template <int MODE>
__global__ __launch_bounds__(kDispBlock) void place_kernel(
    const int32_t* __restrict__ ids, int n, int E, int tile, int tiles,
    const int32_t* __restrict__ tile_hist, int32_t* __restrict__ counts,
    int32_t* __restrict__ offsets, int32_t* __restrict__ perm, int32_t* __restrict__ dest) {
    extern __shared__ __attribute__((aligned(16))) int32_t lds[];
    place_body<MODE>(blockIdx.x, lds, ids, n, E, tile, tiles, tile_hist, counts, offsets, perm, dest);
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
int place_mode(long long n, int E) {
    const TilePlan p = plan_tiles(n);
    if (p.tiles == 1) return kPlaceSingle;
    return static_cast<long long>(p.tiles) * p.tiles * E <= kFuseLimit ? kPlaceFused : kPlaceScanned;
}

int run_scan(int32_t* tile_counts, long long n, int E, int32_t* counts, void* stream) {
    const TilePlan p = plan_tiles(n);
    return launch(scan_kernel, dim3(ceil_div(E, kWave)), dim3(kDispBlock), 0, stream, tile_counts, p.tiles, E,
                  counts);
}

int run_place(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
              int32_t* dest, int32_t* tile_counts, void* stream) {
    const TilePlan p = plan_tiles(n);
    if (p.tiles == 1)
        return launch(place_kernel<kPlaceSingle>, dim3(1), dim3(kDispBlock), place_lds_bytes(kPlaceSingle, E),
                      stream, topk_ids, p.n, E, p.tile, p.tiles, static_cast<const int32_t*>(tile_counts),
                      counts, offsets, perm, dest);
    if (static_cast<long long>(p.tiles) * p.tiles * E <= kFuseLimit)
        return launch(place_kernel<kPlaceFused>, dim3(p.tiles), dim3(kDispBlock), place_lds_bytes(kPlaceFused, E),
                      stream, topk_ids, p.n, E, p.tile, p.tiles, static_cast<const int32_t*>(tile_counts),
                      counts, offsets, perm, dest);
    const int rc = run_scan(tile_counts, n, E, counts, stream);
    if (rc) return rc;
    return launch(place_kernel<kPlaceScanned>, dim3(p.tiles), dim3(kDispBlock), place_lds_bytes(kPlaceScanned, E), stream, topk_ids, p.n, E,
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
