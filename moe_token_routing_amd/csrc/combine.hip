// moe_combine: post-expert RMSNorm of each selected expert row, routing-weight
// scaling and top-k sum, skipping invalid slots.
//
// Method: TensorRT-LLM PR #21356 ("Add the Muse Spark Open decoder fast
// paths"), description, Triton kernel "Post-expert norm and combine" and
// "Routing" (pick order fixes the summation order); TensorRT-LLM PR #21042
// ("Add the Muse Spark Open model"), Description, "MoE".
//
// Design (gfx950): HBM-bound row gathers. Each token's k expert rows are
// loaded in groups of G with 16-byte non-temporal loads spread over the
// token's threads (every wave-wide load covers 1 KB of one row); a slot
// outside [0, R) issues no load at all. The G sums of squares are reduced
// together (v_dot2_f32_bf16 on the packed pairs, then across the token's
// threads), each normalised row is rounded to BF16 two elements at a time
// (v_cvt_pk_bf16_f32) and the weighted rows accumulate in FP32 registers in
// slot order (one FMA per element). That is about six VALU operations per
// element, so the kernel stays under the HBM time. The per-element gain is
// kept in registers when a token fills the block, else staged in LDS once
// per block and read there for every token the block visits; the grid has
// one block per block's worth of tokens, so the hardware hands out tokens
// as blocks finish. Batches of no more tokens than CUs take
// combine_token_kernel: one 1024-thread block per token, or per part of a
// token's row when CUs are left over.
#include <cmath>

#include "launch.hpp"
#include "rows.hpp"

namespace moe {
namespace {

template <int VPT>
struct CombineCfg {
    // rows per group: 64 data VGPRs per thread for narrow rows, 64 for H=8192
    static constexpr int G = VPT >= 8 ? 2 : (VPT >= 4 ? 4 : 8);
};

// TPT = 0: tpt threads per token, any power of two up to kRowBlock, with
// bounds checks. TPT = kWave or kRowBlock: one token per wave or per block
// and every thread owns exactly VPT vectors (H / 8 = VPT TPT). The token,
// its slots and their validity are then the same for the whole wave, so they
// live in scalar registers and the per-vector bounds checks disappear.
template <int VPT, int TPT>
__global__ __launch_bounds__(kRowBlock) void combine_kernel(
    const u32x4* __restrict__ expert_out, int R, const int32_t* __restrict__ slots,
    const float* __restrict__ topk_w, const float* __restrict__ norm_w, float gain_center,
    float eps, int T, int H, int k, int tpt, u32x4* __restrict__ out) {
    constexpr int G = CombineCfg<VPT>::G;
    __shared__ float red[(kRowBlock / kWave) * G];
    // gain = gain_center + norm_w. When a token fills the block (TPT =
    // kRowBlock) and a thread owns at most four vectors, each thread keeps
    // the gains of its own VPT vectors in registers, read once (the block has one token: staging the whole gain
    // row in LDS and reading it back per row had cost the prefill combine
    // 203 against 198 us). Otherwise it is staged once per block: vector v's
    // eight values live as gain_lo[v] (elements 0-3) and gain_hi[v] (4-7), so
    // a wave's 16-byte LDS reads are consecutive.
    constexpr bool GREG = TPT == kRowBlock && VPT <= 4;
    float greg[GREG ? VPT : 1][8];
    if constexpr (GREG) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = static_cast<int>(threadIdx.x) + i * kRowBlock;
            const float4 a = reinterpret_cast<const float4*>(norm_w)[2 * v];
            const float4 b = reinterpret_cast<const float4*>(norm_w)[2 * v + 1];
            greg[i][0] = gain_center + a.x;
            greg[i][1] = gain_center + a.y;
            greg[i][2] = gain_center + a.z;
            greg[i][3] = gain_center + a.w;
            greg[i][4] = gain_center + b.x;
            greg[i][5] = gain_center + b.y;
            greg[i][6] = gain_center + b.z;
            greg[i][7] = gain_center + b.w;
        }
    }
    extern __shared__ float4 gain_lds[];
    const int nvec = H >> 3;
    float4* gain_lo = gain_lds;
    float4* gain_hi = gain_lds + nvec;
    if (!GREG)
    for (int v = threadIdx.x; v < nvec; v += kRowBlock) {
        const float4 a = reinterpret_cast<const float4*>(norm_w)[2 * v];
        const float4 b = reinterpret_cast<const float4*>(norm_w)[2 * v + 1];
        gain_lo[v] = make_float4(gain_center + a.x, gain_center + a.y, gain_center + a.z, gain_center + a.w);
        gain_hi[v] = make_float4(gain_center + b.x, gain_center + b.y, gain_center + b.z, gain_center + b.w);
    }
    if (!GREG) __syncthreads();

    constexpr bool WHOLE = TPT != 0;
    if (WHOLE) tpt = TPT;
    const int tokens_per_block = kRowBlock / tpt;
    // with TPT a multiple of the wave, a wave's lanes share one token
    const int sub = WHOLE ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT)
                          : static_cast<int>(threadIdx.x) / tpt;
    const int tid = static_cast<int>(threadIdx.x) - sub * tpt;
    const float hf = static_cast<float>(H);

    // 64-bit token index: with a block per token the stride is the whole
    // batch, and t0 + stride must not overflow for batches past 2^30 tokens
    const long long stride = static_cast<long long>(gridDim.x) * tokens_per_block;
    for (long long t0 = static_cast<long long>(blockIdx.x) * tokens_per_block; t0 < T; t0 += stride) {
        const int t = static_cast<int>(t0) + sub;
        const bool tok_ok = t < T;
        float acc[VPT][8];
#pragma unroll
        for (int i = 0; i < VPT; ++i)
#pragma unroll
            for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

        for (int j0 = 0; j0 < k; j0 += G) {
            u32x4 x[G][VPT];
            float ss[G];
            bool ok[G];
            float wt[G];
#pragma unroll
            for (int g = 0; g < G; ++g) {
                const int j = j0 + g;
                int r = -1;
                wt[g] = 0.f;
                if (tok_ok && j < k) {
                    r = slots[static_cast<size_t>(t) * k + j];
                    wt[g] = topk_w[static_cast<size_t>(t) * k + j];
                }
                ok[g] = r >= 0 && r < R;
                if (ok[g]) {
                    const u32x4* row = expert_out + static_cast<size_t>(r) * nvec;
#pragma unroll
                    for (int i = 0; i < VPT; ++i) {
                        const int v = tid + i * tpt;
                        if (WHOLE || v < nvec) x[g][i] = load_nt(&row[v]);
                    }
                }
            }
#pragma unroll
            for (int g = 0; g < G; ++g) {
                float s = 0.f;
                if (ok[g]) {
#pragma unroll
                    for (int i = 0; i < VPT; ++i) {
                        if (WHOLE || tid + i * tpt < nvec) {
                            s = dot2_sq(x[g][i].x, s);
                            s = dot2_sq(x[g][i].y, s);
                            s = dot2_sq(x[g][i].z, s);
                            s = dot2_sq(x[g][i].w, s);
                        }
                    }
                }
                ss[g] = s;
            }
            token_sum(ss, tpt, red);
#pragma unroll
            for (int g = 0; g < G; ++g) {
                if (!ok[g]) continue;
                const float rinv = 1.0f / sqrtf(ss[g] / hf + eps);
                const float w = wt[g];
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    const int v = tid + i * tpt;
                    if (!WHOLE && v >= nvec) continue;
                    const uint32_t w4[4] = {x[g][i].x, x[g][i].y, x[g][i].z, x[g][i].w};
                    float gv[8];
                    if constexpr (GREG) {
#pragma unroll
                        for (int q = 0; q < 8; ++q) gv[q] = greg[i][q];
                    } else {
                        const float4 ga = gain_lo[v], gb = gain_hi[v];
                        gv[0] = ga.x;
                        gv[1] = ga.y;
                        gv[2] = ga.z;
                        gv[3] = ga.w;
                        gv[4] = gb.x;
                        gv[5] = gb.y;
                        gv[6] = gb.z;
                        gv[7] = gb.w;
                    }
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const float y0 = (bf16_lo(w4[q]) * gv[2 * q]) * rinv;
                        const float y1 = (bf16_hi(w4[q]) * gv[2 * q + 1]) * rinv;
                        const uint32_t z = cvt_pk_bf16(y0, y1);
                        acc[i][2 * q] = __builtin_fmaf(w, bf16_lo(z), acc[i][2 * q]);
                        acc[i][2 * q + 1] = __builtin_fmaf(w, bf16_hi(z), acc[i][2 * q + 1]);
                    }
                }
            }
        }
        if (tok_ok) {
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const int v = tid + i * tpt;
                if (WHOLE || v < nvec) {
                    u32x4 o;
                    o.x = cvt_pk_bf16(acc[i][0], acc[i][1]);
                    o.y = cvt_pk_bf16(acc[i][2], acc[i][3]);
                    o.z = cvt_pk_bf16(acc[i][4], acc[i][5]);
                    o.w = cvt_pk_bf16(acc[i][6], acc[i][7]);
                    store_nt(o, &out[static_cast<size_t>(t) * nvec + v]);
                }
            }
        }
    }
}

// Batches of no more tokens than CUs, rows of 1024 * VPT vectors: one
// 1024-thread block per token, or S blocks (S = 1, 2 or 4) when CUs are left
// over. Each of the S blocks reads the token's whole rows for the sums of
// squares, but only its S-th of the waves (part `part`) normalises, weights
// and stores, so the per-element work (most of the time at these sizes)
// spreads over S CUs. Block b serves token (b / 8 / S) * 8 + b % 8: the S
// blocks of a token share b % 8 and so an XCD (blocks go to the 8 XCDs in
// turn) and its L2, which serves the repeated row reads.
// Each thread owns VPT vectors, so its gains stay in registers (no LDS stage
// and no barrier before the first row load); lane j of every wave holds pick
// j's slot and weight (k <= 32), so one load brings them all and the first
// rows issue right behind it; the next group's rows are in flight while the
// block adds the current group's sums of squares, and two reduction buffers
// alternate, so a group costs one barrier. The arithmetic and its order are
// those of combine_kernel.
constexpr int kBigBlock = 1024;
constexpr int kXcds = 8;
constexpr int kMaxParts = 4;

template <int VPT>
__global__ __launch_bounds__(kBigBlock) void combine_token_kernel(
    const u32x4* __restrict__ expert_out, int R, const int32_t* __restrict__ slots,
    const float* __restrict__ topk_w, const float* __restrict__ norm_w, float gain_center,
    float eps, int T, int H, int k, int S, u32x4* __restrict__ out) {
    constexpr int G = VPT == 1 ? 8 : 4;   // rows a group: 32 data VGPRs, twice for the next group
    constexpr int kWaves = kBigBlock / kWave;
    __shared__ float red[2][kWaves][G];
    const int round = blockIdx.x / kXcds;
    const int t = (round / S) * kXcds + blockIdx.x % kXcds;
    const int part = round % S;
    if (t >= T) return;
    const int nvec = H >> 3;
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const bool mine = wave / (kWaves / S) == part;   // this wave's vectors are this block's to write
    int pick_r = -1;
    float pick_w = 0.f;
    if (lane < k) {
        pick_r = slots[static_cast<size_t>(t) * k + lane];
        pick_w = topk_w[static_cast<size_t>(t) * k + lane];
    }
    float gv[VPT][8] = {};
    if (mine) {
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = threadIdx.x + i * kBigBlock;
            const float4 a = reinterpret_cast<const float4*>(norm_w)[2 * v];
            const float4 b = reinterpret_cast<const float4*>(norm_w)[2 * v + 1];
            gv[i][0] = gain_center + a.x; gv[i][1] = gain_center + a.y;
            gv[i][2] = gain_center + a.z; gv[i][3] = gain_center + a.w;
            gv[i][4] = gain_center + b.x; gv[i][5] = gain_center + b.y;
            gv[i][6] = gain_center + b.z; gv[i][7] = gain_center + b.w;
        }
    }
    float acc[VPT][8];
#pragma unroll
    for (int i = 0; i < VPT; ++i)
#pragma unroll
        for (int e = 0; e < 8; ++e) acc[i][e] = 0.f;

    // rows of picks j0 .. j0 + G - 1; every lane read happens outside the
    // branches (lanes k .. 63 hold slot -1, and j0 + G - 1 < 64 since k <= 32),
    // so the wait for the picks is taken once and the row loads all stay in
    // flight together
    auto issue = [&](u32x4 (&x)[G][VPT], bool (&ok)[G], int j0) {
        int r[G];
#pragma unroll
        for (int g = 0; g < G; ++g) r[g] = __builtin_amdgcn_readlane(pick_r, j0 + g);
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ok[g] = r[g] >= 0 && r[g] < R;
            if (ok[g]) {
                const u32x4* row = expert_out + static_cast<size_t>(r[g]) * nvec;
#pragma unroll
                for (int i = 0; i < VPT; ++i) x[g][i] = load_nt(&row[threadIdx.x + i * kBigBlock]);
            }
        }
    };
    u32x4 x[G][VPT];
    bool ok[G];
    issue(x, ok, 0);
    int buf = 0;
    for (int j0 = 0; j0 < k; j0 += G, buf ^= 1) {
        u32x4 xn[G][VPT];
        bool okn[G];
        issue(xn, okn, j0 + G);
        float wt[G];
#pragma unroll
        for (int g = 0; g < G; ++g) wt[g] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(pick_w), j0 + g));
        float ss[G];
#pragma unroll
        for (int g = 0; g < G; ++g) {
            float s = 0.f;
            if (ok[g]) {
#pragma unroll
                for (int i = 0; i < VPT; ++i) {
                    s = dot2_sq(x[g][i].x, s);
                    s = dot2_sq(x[g][i].y, s);
                    s = dot2_sq(x[g][i].z, s);
                    s = dot2_sq(x[g][i].w, s);
                }
            }
            ss[g] = wave_sum(s);
        }
        if (lane == 0) {
#pragma unroll
            for (int g = 0; g < G; ++g) red[buf][wave][g] = ss[g];
        }
        __syncthreads();
        // lane g of each wave adds pick j0 + g's wave sums (in wave order)
        // and takes its 1 / rms once; the wave reads the G results back
        float rv = 0.f;
        if (mine && lane < G) {
            float s = red[buf][0][lane];
            for (int w = 1; w < kWaves; ++w) s += red[buf][w][lane];
            rv = 1.0f / sqrtf(s / static_cast<float>(H) + eps);
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            if (!ok[g] || !mine) continue;
            const float rinv = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(rv), g));
#pragma unroll
            for (int i = 0; i < VPT; ++i) {
                const uint32_t w4[4] = {x[g][i].x, x[g][i].y, x[g][i].z, x[g][i].w};
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const float y0 = (bf16_lo(w4[q]) * gv[i][2 * q]) * rinv;
                    const float y1 = (bf16_hi(w4[q]) * gv[i][2 * q + 1]) * rinv;
                    const uint32_t z = cvt_pk_bf16(y0, y1);
                    acc[i][2 * q] = __builtin_fmaf(wt[g], bf16_lo(z), acc[i][2 * q]);
                    acc[i][2 * q + 1] = __builtin_fmaf(wt[g], bf16_hi(z), acc[i][2 * q + 1]);
                }
            }
        }
#pragma unroll
        for (int g = 0; g < G; ++g) {
            ok[g] = okn[g];
#pragma unroll
            for (int i = 0; i < VPT; ++i) x[g][i] = xn[g][i];
        }
    }
    if (!mine) return;
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        u32x4 o;
        o.x = cvt_pk_bf16(acc[i][0], acc[i][1]);
        o.y = cvt_pk_bf16(acc[i][2], acc[i][3]);
        o.z = cvt_pk_bf16(acc[i][4], acc[i][5]);
        o.w = cvt_pk_bf16(acc[i][6], acc[i][7]);
        store_nt(o, &out[static_cast<size_t>(t) * nvec + threadIdx.x + i * kBigBlock]);
    }
}

template <int VPT, int TPT>
int launch_combine(const uint16_t* expert_out, int R, const int32_t* slots, const float* topk_w,
                   const float* norm_w, float gain_center, float eps, int T, int H, int k,
                   const RowGeom& geo, uint16_t* out, void* stream) {
    // One block for each block's worth of tokens, dispatched by the hardware
    // as blocks finish, rather than a resident grid striding over the
    // tokens: at 8192 tokens of 8192, k 8 the combine 213 -> 203 us, at
    // 32768 tokens of 1024, k 22 298 -> 275 us (the gain staging per block
    // reads the gain from L2); the kernel's token loop still covers any grid.
    const int tokens_per_block = kRowBlock / geo.tpt;
    const int grid = ceil_div(T, tokens_per_block);
    // the gain row in LDS, unless the kernel keeps the gains in registers
    const size_t lds = TPT == kRowBlock && VPT <= 4 ? 0 : sizeof(float) * static_cast<size_t>(H);
    return launch(combine_kernel<VPT, TPT>, dim3(grid), dim3(kRowBlock), lds, stream,
                  reinterpret_cast<const u32x4*>(expert_out), R, slots, topk_w, norm_w,
                  gain_center, eps, T, H, k, geo.tpt, reinterpret_cast<u32x4*>(out));
}

}  // namespace
}  // namespace moe

extern "C" int moe_combine(const uint16_t* expert_out, int R, const int32_t* slots,
                           const float* topk_w, const float* norm_w, float gain_center, float eps,
                           int T, int H, int k, uint16_t* out, void* stream) {
    using namespace moe;
    if (T < 0 || R < 0 || k < 1 || k > MOE_MAX_TOPK || H < 8 || H > MOE_MAX_HIDDEN || H % 8 != 0)
        return MOE_ERR_BAD_SHAPE;
    if (static_cast<long long>(T) * k >= (1ll << 31) ||
        static_cast<long long>(R) * (H / 8) >= (1ll << 40))
        return MOE_ERR_BAD_SHAPE;
    if (!std::isfinite(gain_center) || !std::isfinite(eps) || eps < 0.f) return MOE_ERR_BAD_ARG;
    if (T == 0) return MOE_OK;
    if (!slots || !topk_w || !norm_w || !out || (R > 0 && !expert_out)) return MOE_ERR_NULL_ARG;
    if (!all_aligned16(expert_out, slots, topk_w, norm_w, out)) return MOE_ERR_ALIGN;
    RowGeom geo = row_geom(H);
    // no more tokens than CUs and rows of 1024 or 2048 vectors: the token
    // kernel, its row cut in S parts while CUs are left over (at 128 tokens
    // of 8192, k 8: 10.7 -> 7.2 us; at 5 tokens, k 32: 37.7 -> 15.4 us)
    const int cus = device_cu_count();
    if (T <= cus && (geo.nvec == kBigBlock || geo.nvec == 2 * kBigBlock)) {
        const int T8 = ceil_div(T, kXcds) * kXcds;
        int S = 1;
        while (S < kMaxParts && T8 * S * 2 <= cus) S *= 2;
        auto kern = geo.nvec == kBigBlock ? combine_token_kernel<1> : combine_token_kernel<2>;
        return launch(kern, dim3(T8 * S), dim3(kBigBlock), 0, stream, reinterpret_cast<const u32x4*>(expert_out),
                      R, slots, topk_w, norm_w, gain_center, eps, T, H, k, S, reinterpret_cast<u32x4*>(out));
    }
    // rows of at most 128 vectors (H <= 1024): one wave per token, so the
    // token's sums of squares never meet in LDS (measured at H 1024, k 22:
    // 446 -> 395 us); wider rows keep the whole block (one wave per token
    // was slower at H 4096)
    if (geo.nvec <= 2 * kWave && geo.tpt > kWave) {
        geo.tpt = kWave;
        geo.vpt = (geo.nvec + kWave - 1) / kWave;
    }
    int vpt = 1;
    while (vpt < geo.vpt) vpt <<= 1;
    const int tpt_whole = (geo.tpt == kRowBlock || geo.tpt == kWave) && geo.nvec == vpt * geo.tpt ? geo.tpt : 0;
#define MOE_COMBINE(V) (tpt_whole == kRowBlock ? launch_combine<V, kRowBlock>(MOE_COMBINE_ARGS) \
                        : tpt_whole == kWave   ? launch_combine<V, kWave>(MOE_COMBINE_ARGS)     \
                                               : launch_combine<V, 0>(MOE_COMBINE_ARGS))
#define MOE_COMBINE_ARGS expert_out, R, slots, topk_w, norm_w, gain_center, eps, T, H, k, geo, out, stream
    switch (vpt) {
        case 1: return MOE_COMBINE(1);
        case 2: return MOE_COMBINE(2);
        case 4: return MOE_COMBINE(4);
        case 8: return MOE_COMBINE(8);
        default: return MOE_ERR_BAD_SHAPE;
    }
#undef MOE_COMBINE_ARGS
#undef MOE_COMBINE
}
