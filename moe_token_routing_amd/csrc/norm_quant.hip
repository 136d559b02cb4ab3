// moe_norm_quant_nvfp4: RMSNorm of the expert input (one BF16 rounding) fused
// with NVFP4 quantisation: E2M1 codes, E4M3 scales per 16-element block,
// static global scale.
//
// Method: vLLM API docs, vllm.models.muse_spark.nvidia.ops.prepare_trtllm_nvfp4
// (`norm_quant_trtllm_nvfp4`; the per-block arithmetic of
// `_quantize_nvfp4_global_scale`, taken step for step in FP32 with IEEE
// reciprocals); TensorRT-LLM PR #21356, description, "Numerics" (gain centre
// added in FP32, the norm rounds only its result).
//
// The input may also be in the rank-block layout [tp*T, H/tp] that a dim-0
// all-gather of column shards leaves (same docs, module description): each
// thread's vectors keep their rank block for every token, so the layout only
// changes a per-thread row offset computed once.
//
// Design (gfx950): one HBM pass. A row is read once with 16-byte loads into
// registers; its sum of squares is reduced across the token's threads. Each
// lane owns whole 16-element blocks (two neighbouring vectors), so a block's
// maximum, E4M3 scale (hardware FP8 conversion, clamped to saturate) and
// reciprocal are computed once, and its 16 codes (hardware FP4 conversion)
// leave as one 8-byte store, its scale as one byte.
//
// When a block visits several tokens and a token fills whole waves or the
// whole block, the next token's row is copied into LDS by global_load_lds
// while this token is reduced and quantised, so a block always has a row in
// flight and the copy costs no registers. Each wave reads back only the LDS
// slots its own copies wrote, so a wave waits for its own copies and
// nothing else; the token's sum of squares crosses waves through a
// double-buffered LDS slot with one barrier that does not wait for the
// copies in flight. Same arithmetic, same order.
#include <cmath>

#include "launch.hpp"
#include "nvfp4.hpp"
#include "rows.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float round_to_bf16(float f) {
    return __uint_as_float(f32_to_bf16_rne(f) << 16);
}

// One 16-element block: normalise (x * gain) * rinv, round once to BF16,
// take the block maximum, its E4M3 scale byte and the 16 E2M1 codes (element
// 2j in the low nibble of byte j). Returns the codes, the scale byte in *sf.
__device__ __forceinline__ uint2 encode_block(const uint32_t (&xw)[8], const float (&gain)[16], float rinv,
                                              float gs, float rcp_gs, uint32_t* sf_out) {
    constexpr float kRcp6 = 1.0f / 6.0f;
    // normalised pairs, rounded once to BF16 (packed)
    uint32_t yp[8];
#pragma unroll
    for (int q = 0; q < 8; ++q)
        yp[q] = cvt_pk_bf16((bf16_lo(xw[q]) * gain[2 * q]) * rinv, (bf16_hi(xw[q]) * gain[2 * q + 1]) * rinv);
    // block maximum of |y|: the magnitude bits of non-negative BF16
    // values order like integers, and a NaN magnitude exceeds inf.
    uint32_t m = packed_max_u16(yp[0] & 0x7FFF7FFFu, yp[1] & 0x7FFF7FFFu);
#pragma unroll
    for (int q = 2; q < 8; ++q) m = packed_max_u16(m, yp[q] & 0x7FFF7FFFu);
    const uint32_t mbits = max(m & 0xFFFFu, m >> 16);
    const float bmax = __uint_as_float(mbits << 16);
    const float tq = bmax * kRcp6;
    const float s = gs * tq;
    const uint32_t sf = e4m3_scale_code(s);
    const float sf_f = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sf), 0);
    const float d = sf_f * rcp_gs;
    const float outs = (sf_f != 0.f) ? 1.0f / d : 0.f;
    uint32_t w0 = 0, w1 = 0;
    if (mbits < 0x7F80u && fabsf(outs) < INFINITY) {
        // q = y * out with -0 turned into +0 (fma with a +0 addend, one
        // rounding); the hardware E2M1 conversion with unit scale rounds
        // finite values to nearest even and saturates.
        w0 = fp4_pair<0>(w0, yp[0], outs);
        w0 = fp4_pair<1>(w0, yp[1], outs);
        w0 = fp4_pair<2>(w0, yp[2], outs);
        w0 = fp4_pair<3>(w0, yp[3], outs);
        w1 = fp4_pair<0>(w1, yp[4], outs);
        w1 = fp4_pair<1>(w1, yp[5], outs);
        w1 = fp4_pair<2>(w1, yp[6], outs);
        w1 = fp4_pair<3>(w1, yp[7], outs);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0 |= e2m1_code(bf16_lo(yp[q]) * outs) << (8 * q);
            w0 |= e2m1_code(bf16_hi(yp[q]) * outs) << (8 * q + 4);
            w1 |= e2m1_code(bf16_lo(yp[q + 4]) * outs) << (8 * q);
            w1 |= e2m1_code(bf16_hi(yp[q + 4]) * outs) << (8 * q + 4);
        }
    }
    *sf_out = sf;
    return make_uint2(w0, w1);
}

// gains of one 16-element block: centre + weight, in FP32
__device__ __forceinline__ void load_gains(const float* norm_w, int b, float gain_center, float (&gain)[16]) {
    const float4* g4 = reinterpret_cast<const float4*>(norm_w) + 4 * b;
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float4 a = g4[q];
        gain[4 * q] = gain_center + a.x;
        gain[4 * q + 1] = gain_center + a.y;
        gain[4 * q + 2] = gain_center + a.z;
        gain[4 * q + 3] = gain_center + a.w;
    }
}

// One lane quantises whole 16-element blocks: block b of a row is two
// neighbouring 16-byte vectors, so its scale is computed once, by the lane
// that holds it. A 256-thread block serves 256 / tpt tokens, tpt threads per
// token (tpt = the power of two >= H/16, at most 256), BPT blocks per thread.
// TPT = 0: tpt threads per token, with bounds checks. TPT = kWave or
// kRowBlock: one token per wave or per block and exactly BPT blocks per
// thread (H / 16 = BPT TPT), so the token is the same for the whole wave
// and the per-block bounds checks disappear.
template <int BPT, int TPT>
__global__ __launch_bounds__(kRowBlock) void norm_quant_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center, float eps,
    const float* __restrict__ global_scale, int T, int H, int shard8, int tpt,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    __shared__ float red[kRowBlock / kWave];
    const int nblk = H >> 4;
    constexpr bool WHOLE = TPT != 0;
    if (WHOLE) tpt = TPT;
    const int tokens_per_block = kRowBlock / tpt;
    // with TPT a multiple of the wave, a wave's lanes share one token
    const int sub = WHOLE ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT)
                          : static_cast<int>(threadIdx.x) / tpt;
    const int tid = static_cast<int>(threadIdx.x) - sub * tpt;
    const float hf = static_cast<float>(H);
    const float gs = *global_scale;
    const float rcp_gs = 1.0f / gs;
    // gains of this thread's blocks, and where block b of token t starts:
    // src[i] + t * shard8 (16-byte units; both vectors of a block lie in one
    // rank block since shard % 16 == 0)
    float gain[BPT][16];
    size_t src[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = tid + i * tpt;
        const int v = 2 * b;
        const int rb = v / shard8;
        src[i] = static_cast<size_t>(rb) * T * shard8 + (v - rb * shard8);
#pragma unroll
        for (int e = 0; e < 16; ++e) gain[i][e] = 0.f;
        if (WHOLE || b < nblk) load_gains(norm_w, b, gain_center, gain[i]);
    }

    for (int t0 = blockIdx.x * tokens_per_block; t0 < T; t0 += gridDim.x * tokens_per_block) {
        const int t = t0 + sub;
        const bool tok_ok = t < T;
        uint32_t xw[BPT][8];   // block i: 16 BF16 values as 8 packed pairs
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            u32x4 a = u32x4{0u, 0u, 0u, 0u}, c = u32x4{0u, 0u, 0u, 0u};
            if (WHOLE ? tok_ok : (tok_ok && tid + i * tpt < nblk)) {
                const u32x4* p = &x[src[i] + static_cast<size_t>(t) * shard8];
                a = load_nt(p);
                c = load_nt(p + 1);
            }
            xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
            xw[i][4] = c.x; xw[i][5] = c.y; xw[i][6] = c.z; xw[i][7] = c.w;
        }
        float ss[1] = {0.f};
#pragma unroll
        for (int i = 0; i < BPT; ++i)
#pragma unroll
            for (int q = 0; q < 8; ++q) ss[0] = dot2_sq(xw[i][q], ss[0]);
        token_sum(ss, tpt, red);
        const float rinv = 1.0f / sqrtf(ss[0] / hf + eps);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + i * tpt;
            uint32_t sf;
            const uint2 codes = encode_block(xw[i], gain[i], rinv, gs, rcp_gs, &sf);
            if (WHOLE ? tok_ok : (tok_ok && b < nblk)) {
                packed[static_cast<size_t>(t) * nblk + b] = codes;
                scales[static_cast<size_t>(t) * nblk + b] = static_cast<uint8_t>(sf);
            }
        }
    }
}

// 16 bytes per lane from global memory into LDS (global_load_lds_dwordx4):
// lane l of the wave writes dst + 16 l, where dst is the wave's base.
__device__ __forceinline__ void copy16_to_lds(const u32x4* src, u32x4* dst) {
    __builtin_amdgcn_global_load_lds(reinterpret_cast<const void*>(src), reinterpret_cast<void*>(dst), 16, 0, 0);
}
// s_waitcnt vmcnt(0): this wave's copies (and stores) have landed
__device__ __forceinline__ void wait_copies() {
    __builtin_amdgcn_s_waitcnt(0x70);
    asm volatile("" ::: "memory");
}
// s_waitcnt lgkmcnt(0): this wave's LDS accesses are done
__device__ __forceinline__ void wait_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    asm volatile("" ::: "memory");
}
// LDS writes done, then a barrier that leaves global copies in flight
__device__ __forceinline__ void barrier_lds() {
    __builtin_amdgcn_s_waitcnt(0xC07F);
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// The TPT = kWave or kRowBlock case of norm_quant_kernel for blocks that
// visit several tokens: the next token of each wave is copied into LDS while
// this one is reduced and quantised. stage[2i + j][thread] holds vector j of
// the thread's block i; a wave's copies write only its own 64 slots of each
// row, which it alone reads back.
template <int BPT, int TPT>
__global__ __launch_bounds__(kRowBlock) void norm_quant_staged_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center, float eps,
    const float* __restrict__ global_scale, int T, int H, int shard8,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    static_assert(TPT == kWave || TPT == kRowBlock, "whole waves or the whole block per token");
    __shared__ float red[2][kRowBlock / kWave];
    __shared__ u32x4 stage[2 * BPT][kRowBlock];
    constexpr int nblk = BPT * TPT;
    constexpr int tokens_per_block = kRowBlock / TPT;
    const int sub = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT);
    const int tid = static_cast<int>(threadIdx.x) - sub * TPT;
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    const int wbase = wave * kWave;
    const float hf = static_cast<float>(H);
    const float gs = *global_scale;
    const float rcp_gs = 1.0f / gs;
    float gain[BPT][16];
    size_t src[BPT];
#pragma unroll
    for (int i = 0; i < BPT; ++i) {
        const int b = tid + i * TPT;
        const int v = 2 * b;
        const int rb = v / shard8;
        src[i] = static_cast<size_t>(rb) * T * shard8 + (v - rb * shard8);
        load_gains(norm_w, b, gain_center, gain[i]);
    }
    const int step = gridDim.x * tokens_per_block;
    int t = blockIdx.x * tokens_per_block + sub;
    if (t < T) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const u32x4* p = &x[src[i] + static_cast<size_t>(t) * shard8];
            copy16_to_lds(p, &stage[2 * i][wbase]);
            copy16_to_lds(p + 1, &stage[2 * i + 1][wbase]);
        }
    }
    int par = 0;
    // block-uniform trip count (every wave reaches every barrier)
    for (int t0 = blockIdx.x * tokens_per_block; t0 < T; t0 += step, t += step, par ^= 1) {
        // uniform in the wave; with one token per block always true here
        const bool tok_ok = TPT == kRowBlock || t < T;
        wait_copies();
        uint32_t xw[BPT][8];
        float ss = 0.f;
        if (tok_ok) {
#pragma unroll
            for (int i = 0; i < BPT; ++i) {
                const u32x4 a = stage[2 * i][threadIdx.x], c = stage[2 * i + 1][threadIdx.x];
                xw[i][0] = a.x; xw[i][1] = a.y; xw[i][2] = a.z; xw[i][3] = a.w;
                xw[i][4] = c.x; xw[i][5] = c.y; xw[i][6] = c.z; xw[i][7] = c.w;
            }
#pragma unroll
            for (int i = 0; i < BPT; ++i)
#pragma unroll
                for (int q = 0; q < 8; ++q) ss = dot2_sq(xw[i][q], ss);
            // the wave's slots are read back: copy its next token into them
            wait_lds();
            const int tn = t + step;
            if (tn < T) {
#pragma unroll
                for (int i = 0; i < BPT; ++i) {
                    const u32x4* p = &x[src[i] + static_cast<size_t>(tn) * shard8];
                    copy16_to_lds(p, &stage[2 * i][wbase]);
                    copy16_to_lds(p + 1, &stage[2 * i + 1][wbase]);
                }
            }
        }
        ss = wave_sum(ss);
        if (TPT == kRowBlock) {
            // partial sums added in wave order, as token_sum does
            if (__lane_id() == 0) red[par][wave] = ss;
            barrier_lds();
            ss = red[par][0];
#pragma unroll
            for (int w = 1; w < kRowBlock / kWave; ++w) ss += red[par][w];
        }
        if (!tok_ok) continue;
        const float rinv = 1.0f / sqrtf(ss / hf + eps);
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + i * TPT;
            uint32_t sf;
            const uint2 codes = encode_block(xw[i], gain[i], rinv, gs, rcp_gs, &sf);
            packed[static_cast<size_t>(t) * nblk + b] = codes;
            scales[static_cast<size_t>(t) * nblk + b] = static_cast<uint8_t>(sf);
        }
    }
}

struct BlockGeom {
    int tpt;   // threads per token (power of two, <= 256)
    int bpt;   // 16-element blocks per thread
};

inline BlockGeom block_geom(int H) {
    const int nblk = H / 16;
    BlockGeom g;
    g.tpt = 1;
    while (g.tpt < nblk && g.tpt < kRowBlock) g.tpt <<= 1;
    g.bpt = (nblk + g.tpt - 1) / g.tpt;
    return g;
}

template <int BPT, int TPT>
int launch_norm_quant(const uint16_t* x, const float* norm_w, float gain_center, float eps,
                      const float* global_scale, int T, int H, int shard, const BlockGeom& geo,
                      uint8_t* packed, uint8_t* scales, void* stream) {
    const int tokens_per_block = kRowBlock / geo.tpt;
    const int needed = ceil_div(T, tokens_per_block);
    // as many blocks as fit on the GPU at once; each loops over its tokens
    const int cap = device_cu_count() * resident_blocks(norm_quant_kernel<BPT, TPT>, kRowBlock, 0);
    if constexpr (TPT != 0) {
        // blocks that visit several tokens copy each next row in ahead
        const int cap_staged =
            device_cu_count() * resident_blocks(norm_quant_staged_kernel<BPT, TPT>, kRowBlock, 0);
        if (needed > cap_staged)
            return launch(norm_quant_staged_kernel<BPT, TPT>, dim3(cap_staged), dim3(kRowBlock), 0, stream,
                          reinterpret_cast<const u32x4*>(x), norm_w, gain_center, eps, global_scale, T, H,
                          shard / 8, reinterpret_cast<uint2*>(packed), scales);
    }
    const int grid = needed < cap ? needed : cap;
    return launch(norm_quant_kernel<BPT, TPT>, dim3(grid), dim3(kRowBlock), 0, stream,
                  reinterpret_cast<const u32x4*>(x), norm_w, gain_center, eps, global_scale, T, H,
                  shard / 8, geo.tpt, reinterpret_cast<uint2*>(packed), scales);
}

}  // namespace
}  // namespace moe

extern "C" int moe_norm_quant_nvfp4_rank_block(const uint16_t* x, int shard, const float* norm_w,
                                               float gain_center, float eps, const float* global_scale,
                                               int T, int H, uint8_t* packed, uint8_t* scales,
                                               void* stream) {
    using namespace moe;
    if (T < 0 || H < 16 || H > MOE_MAX_HIDDEN || H % 16 != 0) return MOE_ERR_BAD_SHAPE;
    if (shard < 16 || shard > H || shard % 16 != 0 || H % shard != 0) return MOE_ERR_BAD_SHAPE;
    if (!std::isfinite(gain_center) || !std::isfinite(eps) || eps < 0.f) return MOE_ERR_BAD_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !norm_w || !global_scale || !packed || !scales) return MOE_ERR_NULL_ARG;
    if (!all_aligned16(x, norm_w, packed, scales)) return MOE_ERR_ALIGN;
    const BlockGeom geo = block_geom(H);
    const int tpt_whole =
        (geo.tpt == kRowBlock || geo.tpt == kWave) && H / 16 == geo.bpt * geo.tpt ? geo.tpt : 0;
#define MOE_NQ_ARGS x, norm_w, gain_center, eps, global_scale, T, H, shard, geo, packed, scales, stream
#define MOE_NQ(B) (tpt_whole == kRowBlock ? launch_norm_quant<B, kRowBlock>(MOE_NQ_ARGS) \
                   : tpt_whole == kWave   ? launch_norm_quant<B, kWave>(MOE_NQ_ARGS)     \
                                          : launch_norm_quant<B, 0>(MOE_NQ_ARGS))
    switch (geo.bpt) {
        case 1: return MOE_NQ(1);
        case 2: return MOE_NQ(2);
        case 3: return MOE_NQ(3);
        case 4: return MOE_NQ(4);
        default: return MOE_ERR_BAD_SHAPE;
    }
#undef MOE_NQ
#undef MOE_NQ_ARGS
}

extern "C" int moe_norm_quant_nvfp4(const uint16_t* x, const float* norm_w, float gain_center,
                                    float eps, const float* global_scale, int T, int H,
                                    uint8_t* packed, uint8_t* scales, void* stream) {
    if (H < 16 || H % 16 != 0) return MOE_ERR_BAD_SHAPE;
    return moe_norm_quant_nvfp4_rank_block(x, H, norm_w, gain_center, eps, global_scale, T, H, packed,
                                           scales, stream);
}
