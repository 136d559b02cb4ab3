// Steps of moe_dispatch shared with the fused route + dispatch entry point
// (moe_route_dispatch), whose selection counts the tile histograms itself.
#pragma once

#include <stdint.h>

namespace moe {

// The dispatch's tiles of slots: `tiles` tiles of `tile` slots (a multiple
// of 256; the last may be partial). Slot f = t k + j belongs to tile f / tile.
struct DispatchTiles {
    int tiles;
    int tile;
};
DispatchTiles dispatch_tiles(long long n);

// moe_dispatch's argument checks (before any launch); a moe_status.
int check_dispatch(const int32_t* topk_ids, int T, int k, int E, const int32_t* counts, const int32_t* offsets,
                   const int32_t* perm, const int32_t* dest);

// counts and offsets of a dispatch with no slots: all zero.
int run_dispatch_empty(int32_t* counts, int32_t* offsets, int E, void* stream);

// Zeroes n int32 with a kernel.
int run_clear(int32_t* p, long long n, void* stream);

// The dispatch of n = T k slots given their tile histograms
// (tile_counts[tiles][E], the valid ids of each tile counted; unused with
// one tile): expert totals, offsets, perm and dest as moe_dispatch defines
// them. tile_counts may be overwritten.
int run_place(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets, int32_t* perm,
              int32_t* dest, int32_t* tile_counts, void* stream);

}  // namespace moe
