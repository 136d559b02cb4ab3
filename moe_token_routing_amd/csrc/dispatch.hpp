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

// The place step's form for n slots over E experts (a PlaceMode of
// place.hpp: 0 after a separate column scan, 1 summing the tile histograms
// itself, 2 one tile), and that column scan.
int place_mode(long long n, int E);
int run_scan(int32_t* tile_counts, long long n, int E, int32_t* counts, void* stream);

// moe_norm_quant_nvfp4's argument checks (contiguous input), before any launch.
int check_norm_quant(const uint16_t* x, const float* norm_w, float gain_center, float eps,
                     const float* global_scale, int T, int H, const uint8_t* packed, const uint8_t* scales);

// run_place, then moe_norm_quant_nvfp4 of x [T,H]: in one launch when the
// shapes allow (blocks of the place step beside blocks of the staged norm +
// quant), else one after the other. Same outputs either way.
int run_place_norm_quant(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* dest, int32_t* tile_counts, const uint16_t* x,
                         const float* norm_w, float gain_center, float eps, const float* global_scale, int T, int H,
                         uint8_t* packed, uint8_t* scales, void* stream);

}  // namespace moe
