// Row layout shared by the row-streaming kernels (combine, norm + quant).
//
// A row of H BF16 values is split into H/8 vectors of 8 values (16 bytes).
// `tpt` threads serve one token: thread `tid` of the token owns vectors
// tid, tid + tpt, tid + 2*tpt, ... (at most VPT of them), so each vector load
// of a wave covers 64 consecutive 16-byte pieces of a row. When a row has at
// least 256 vectors, tpt = 256 (one block per token); otherwise tpt is the
// next power of two >= H/8 and a 256-thread block serves 256/tpt tokens.
#pragma once

#include "common.hpp"

namespace moe {

constexpr int kRowBlock = 256;

struct RowGeom {
    int nvec;   // vectors per row (H / 8)
    int tpt;    // threads per token (power of two, <= 256)
    int vpt;    // vectors per thread, ceil(nvec / tpt)
};

inline RowGeom row_geom(int H) {
    RowGeom g;
    g.nvec = H / 8;
    int t = 1;
    while (t < g.nvec && t < kRowBlock) t <<= 1;
    g.tpt = t;
    g.vpt = (g.nvec + t - 1) / t;
    return g;
}

// Sum of `v` over the tpt threads of one token. Threads of a token are
// contiguous; tpt is a power of two. When a token spans several waves
// (tpt = 128 or 256) the waves meet in LDS: `red` must hold
// (kRowBlock / 64) * N floats, and every thread of the block must call this
// (it holds barriers). The partial sums are added in wave order, so the
// result does not depend on timing.
template <int N>
__device__ __forceinline__ void token_sum(float (&v)[N], int tpt, float* red) {
    if (tpt <= kWave) {
#pragma unroll
        for (int i = 0; i < N; ++i) v[i] = group_sum(v[i], tpt);
        return;
    }
#pragma unroll
    for (int i = 0; i < N; ++i) v[i] = wave_sum(v[i]);
    const int wave = threadIdx.x / kWave;
    const int wpt = tpt / kWave;
    const int w0 = (wave / wpt) * wpt;
    if (__lane_id() == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i) red[wave * N + i] = v[i];
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float s = red[w0 * N + i];
        for (int w = 1; w < wpt; ++w) s += red[(w0 + w) * N + i];
        v[i] = s;
    }
    __syncthreads();
}

}  // namespace moe
