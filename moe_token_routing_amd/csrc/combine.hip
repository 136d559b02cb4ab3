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
// staged in LDS once per block and read there for every token the block
// visits (grid-stride loop). With no more tokens than CUs, one 1024-thread
// block serves each token.
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
// BLOCK = kBigBlock (TPT = BLOCK): one token per 1024-thread block, for
// batches with no more tokens than CUs. A token then has a whole CU, four
// waves per SIMD, each thread a quarter of the vectors and so a quarter of
// the per-element work (a wave64 VALU operation holds a SIMD four cycles),
// and with one vector a thread all k rows load in one group.
constexpr int kBigBlock = 1024;

template <int VPT, int TPT, int BLOCK = kRowBlock>
__global__ __launch_bounds__(BLOCK) void combine_kernel(
    const u32x4* __restrict__ expert_out, int R, const int32_t* __restrict__ slots,
    const float* __restrict__ topk_w, const float* __restrict__ norm_w, float gain_center,
    float eps, int T, int H, int k, int tpt, u32x4* __restrict__ out) {
    static_assert(BLOCK == kRowBlock || TPT == BLOCK, "the big block serves one token");
    // (the big block's 128 registers a thread hold four rows of a vector)
    constexpr int G = BLOCK == kRowBlock ? CombineCfg<VPT>::G : (VPT == 1 ? 4 : 2);
    __shared__ float red[(BLOCK / kWave) * G];
    // gain = gain_center + norm_w, staged once per block. Vector v's eight
    // values live as gain_lo[v] (elements 0-3) and gain_hi[v] (4-7), so a
    // wave's 16-byte LDS reads are consecutive.
    extern __shared__ float4 gain_lds[];
    const int nvec = H >> 3;
    float4* gain_lo = gain_lds;
    float4* gain_hi = gain_lds + nvec;
    for (int v = threadIdx.x; v < nvec; v += BLOCK) {
        const float4 a = reinterpret_cast<const float4*>(norm_w)[2 * v];
        const float4 b = reinterpret_cast<const float4*>(norm_w)[2 * v + 1];
        gain_lo[v] = make_float4(gain_center + a.x, gain_center + a.y, gain_center + a.z, gain_center + a.w);
        gain_hi[v] = make_float4(gain_center + b.x, gain_center + b.y, gain_center + b.z, gain_center + b.w);
    }
    __syncthreads();

    constexpr bool WHOLE = TPT != 0;
    if (WHOLE) tpt = TPT;
    const int tokens_per_block = BLOCK / tpt;
    // with TPT a multiple of the wave, a wave's lanes share one token
    const int sub = WHOLE ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT)
                          : static_cast<int>(threadIdx.x) / tpt;
    const int tid = static_cast<int>(threadIdx.x) - sub * tpt;
    const float hf = static_cast<float>(H);

    for (int t0 = blockIdx.x * tokens_per_block; t0 < T; t0 += gridDim.x * tokens_per_block) {
        const int t = t0 + sub;
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
                    const float4 ga = gain_lo[v], gb = gain_hi[v];
                    const float gv[8] = {ga.x, ga.y, ga.z, ga.w, gb.x, gb.y, gb.z, gb.w};
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

template <int VPT, int TPT, int BLOCK = kRowBlock>
int launch_combine(const uint16_t* expert_out, int R, const int32_t* slots, const float* topk_w,
                   const float* norm_w, float gain_center, float eps, int T, int H, int k,
                   const RowGeom& geo, uint16_t* out, void* stream) {
    const int tokens_per_block = BLOCK / geo.tpt;
    const int needed = ceil_div(T, tokens_per_block);
    const size_t lds = sizeof(float) * static_cast<size_t>(H);
    const int cap = device_cu_count() * resident_blocks(combine_kernel<VPT, TPT, BLOCK>, BLOCK, lds);
    const int grid = needed < cap ? needed : cap;
    return launch(combine_kernel<VPT, TPT, BLOCK>, dim3(grid), dim3(BLOCK), lds, stream,
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
    // no more tokens than CUs and rows of whole 1024-vector multiples: one
    // 1024-thread block per token (at 128 tokens of 8192: 16.2 -> 13.8 us)
    if (T <= device_cu_count() && geo.nvec % kBigBlock == 0 && geo.nvec / kBigBlock <= 2) {
        geo.tpt = kBigBlock;
        geo.vpt = geo.nvec / kBigBlock;
        if (geo.vpt == 1)
            return launch_combine<1, kBigBlock, kBigBlock>(expert_out, R, slots, topk_w, norm_w, gain_center, eps,
                                                          T, H, k, geo, out, stream);
        return launch_combine<2, kBigBlock, kBigBlock>(expert_out, R, slots, topk_w, norm_w, gain_center, eps, T,
                                                      H, k, geo, out, stream);
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
