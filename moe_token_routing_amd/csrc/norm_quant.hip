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
// leave as one 8-byte store, its scale as one byte. The reciprocal of a
// block's scale takes at most 256 values per call (one per E4M3 byte), so
// each block of threads computes them once into an LDS table. For tokens
// whose sum of squares and rinv are finite, with finite gains (the usual
// case), the block maximum comes from the unrounded products (one v_max3_f32
// per pair) and each value is rounded to BF16 in FP32 layout by one
// conversion; other tokens take the general path. Both give the same bytes.
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

#include "dispatch.hpp"
#include "launch.hpp"
#include "nvfp4.hpp"
#include "place.hpp"
#include "rows.hpp"

namespace moe {
namespace {

// RN to BF16 of an FP32 value, returned as the FP32 value it represents
// (one v_cvt_pk_bf16_f32 with a zero low half; v must not be NaN).
__device__ __forceinline__ float bf16_round(float v) { return __uint_as_float(cvt_pk_bf16(0.f, v)); }

// One 16-element block: normalise (x * gain) * rinv, round once to BF16,
// take the block maximum, its E4M3 scale byte and the 16 E2M1 codes (element
// 2j in the low nibble of byte j). Returns the codes, the scale byte in *sf.
// outs_of[sf] is the block's 1 / (E4M3 value of sf * RN(1 / gs)) (0 when that
// value is 0), precomputed with the same IEEE operations for every byte.
// FINITE: the caller has shown that no normalised value can be NaN (finite
// input and gains, finite rinv), so the block maximum is taken over the
// unrounded |v| (v_max3_f32) and rounded once: RN to BF16 is monotone and
// symmetric, so RN(max |v|) = max |RN(v)|, the same value as the general
// path's maximum over the rounded BF16 magnitudes (which also orders NaN).
template <bool FINITE>
__device__ __forceinline__ uint2 encode_block(const uint32_t (&xw)[8], const float (&gain)[16], float rinv,
                                              float gs, const float* outs_of, uint32_t* sf_out) {
    constexpr float kRcp6 = 1.0f / 6.0f;
    float y[16];   // the normalised values rounded to BF16, as FP32
    uint32_t mbits;
    if constexpr (FINITE) {
        float vmax = 0.f;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const float v0 = (bf16_lo(xw[q]) * gain[2 * q]) * rinv;
            const float v1 = (bf16_hi(xw[q]) * gain[2 * q + 1]) * rinv;
            vmax = fmaxf(fmaxf(vmax, fabsf(v0)), fabsf(v1));   // v_max3_f32 with |.| modifiers
            y[2 * q] = bf16_round(v0);
            y[2 * q + 1] = bf16_round(v1);
        }
        mbits = cvt_pk_bf16(0.f, vmax) >> 16;
    } else {
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
        mbits = max(m & 0xFFFFu, m >> 16);
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            y[2 * q] = bf16_lo(yp[q]);
            y[2 * q + 1] = bf16_hi(yp[q]);
        }
    }
    const float bmax = __uint_as_float(mbits << 16);
    const float tq = bmax * kRcp6;
    const float s = gs * tq;
    const uint32_t sf = e4m3_scale_code(s);
    const float outs = outs_of[sf];
    uint32_t w0 = 0, w1 = 0;
    if (mbits < 0x7F80u && fabsf(outs) < INFINITY) {
        // q = y * out with -0 turned into +0 (fma with a +0 addend, one
        // rounding); the hardware E2M1 conversion with unit scale rounds
        // finite values to nearest even and saturates.
        w0 = fp4_pair<0>(w0, y[0], y[1], outs);
        w0 = fp4_pair<1>(w0, y[2], y[3], outs);
        w0 = fp4_pair<2>(w0, y[4], y[5], outs);
        w0 = fp4_pair<3>(w0, y[6], y[7], outs);
        w1 = fp4_pair<0>(w1, y[8], y[9], outs);
        w1 = fp4_pair<1>(w1, y[10], y[11], outs);
        w1 = fp4_pair<2>(w1, y[12], y[13], outs);
        w1 = fp4_pair<3>(w1, y[14], y[15], outs);
    } else {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            w0 |= e2m1_code(y[2 * q] * outs) << (8 * q);
            w0 |= e2m1_code(y[2 * q + 1] * outs) << (8 * q + 4);
            w1 |= e2m1_code(y[8 + 2 * q] * outs) << (8 * q);
            w1 |= e2m1_code(y[8 + 2 * q + 1] * outs) << (8 * q + 4);
        }
    }
    *sf_out = sf;
    return make_uint2(w0, w1);
}

// outs_of[c] for every E4M3 byte c (one entry per thread of a 256-thread
// block, then a barrier): 1 / (value(c) * rcp_gs), IEEE division, 0 when the
// value is 0; NaN for the NaN codes.
__device__ __forceinline__ void fill_outs_table(float* outs_of, float rcp_gs) {
    static_assert(kRowBlock == 256, "one table entry per thread");
    const int c = threadIdx.x;
    const float sf_f = __builtin_amdgcn_cvt_f32_fp8(c, 0);
    const float d = sf_f * rcp_gs;
    outs_of[c] = (sf_f != 0.f) ? 1.0f / d : 0.f;
    __syncthreads();
}

// Whether every gain is finite (then finite input and a finite rinv give
// no NaN among the normalised values).
template <int BPT>
__device__ __forceinline__ bool gains_finite(const float (&gain)[BPT][16]) {
    bool ok = true;
#pragma unroll
    for (int i = 0; i < BPT; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) ok = ok && fabsf(gain[i][e]) <= 3.40282347e38f;
    return ok;
}

// 1 / sqrt(ss / H + eps), IEEE operations; ss / H as a product with 1 / H
// when H is a power of two (both are the correctly rounded quotient).
__device__ __forceinline__ float rms_inverse(float ss, int H, float hf, float inv_h, float eps) {
    const float mean = (H & (H - 1)) == 0 ? ss * inv_h : ss / hf;
    return 1.0f / sqrtf(mean + eps);
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
__device__ __forceinline__ void norm_quant_body(
    int blk, int nblocks, const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center,
    float eps, const float* __restrict__ global_scale, int T, int H, int shard8, int tpt,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    __shared__ float red[kRowBlock / kWave];
    __shared__ float outs_of[256];
    const int nblk = H >> 4;
    constexpr bool WHOLE = TPT != 0;
    if (WHOLE) tpt = TPT;
    const int tokens_per_block = kRowBlock / tpt;
    // with TPT a multiple of the wave, a wave's lanes share one token
    const int sub = WHOLE ? __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT)
                          : static_cast<int>(threadIdx.x) / tpt;
    const int tid = static_cast<int>(threadIdx.x) - sub * tpt;
    const float hf = static_cast<float>(H);
    const float inv_h = 1.0f / hf;
    const float gs = *global_scale;
    const float rcp_gs = 1.0f / gs;
    fill_outs_table(outs_of, rcp_gs);
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
    const bool gok = gains_finite<BPT>(gain);

    for (int t0 = blk * tokens_per_block; t0 < T; t0 += nblocks * tokens_per_block) {
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
        const float rinv = rms_inverse(ss[0], H, hf, inv_h, eps);
        const bool finite = gok && ss[0] <= 3.40282347e38f && rinv <= 3.40282347e38f;
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + i * tpt;
            uint32_t sf;
            const uint2 codes = finite ? encode_block<true>(xw[i], gain[i], rinv, gs, outs_of, &sf)
                                       : encode_block<false>(xw[i], gain[i], rinv, gs, outs_of, &sf);
            if (WHOLE ? tok_ok : (tok_ok && b < nblk)) {
                packed[static_cast<size_t>(t) * nblk + b] = codes;
                scales[static_cast<size_t>(t) * nblk + b] = static_cast<uint8_t>(sf);
            }
        }
    }
}

template <int BPT, int TPT>
__global__ __launch_bounds__(kRowBlock) void norm_quant_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center, float eps,
    const float* __restrict__ global_scale, int T, int H, int shard8, int tpt,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    norm_quant_body<BPT, TPT>(blockIdx.x, gridDim.x, x, norm_w, gain_center, eps, global_scale, T, H, shard8, tpt,
                              packed, scales);
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
// (the kernel's body as a device function of its block index `blk` among
// `nblocks`, so that it can also run beside other work in one launch)
template <int BPT, int TPT>
__device__ __forceinline__ void norm_quant_staged_body(
    int blk, int nblocks, const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center,
    float eps, const float* __restrict__ global_scale, int T, int H, int shard8,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    static_assert(TPT == kWave || TPT == kRowBlock, "whole waves or the whole block per token");
    __shared__ float red[2][kRowBlock / kWave];
    __shared__ float outs_of[256];
    __shared__ u32x4 stage[2 * BPT][kRowBlock];
    constexpr int nblk = BPT * TPT;
    constexpr int tokens_per_block = kRowBlock / TPT;
    const int sub = __builtin_amdgcn_readfirstlane(static_cast<int>(threadIdx.x) / TPT);
    const int tid = static_cast<int>(threadIdx.x) - sub * TPT;
    const int wave = static_cast<int>(threadIdx.x) / kWave;
    const int wbase = wave * kWave;
    const float hf = static_cast<float>(H);
    const float inv_h = 1.0f / hf;
    const float gs = *global_scale;
    const float rcp_gs = 1.0f / gs;
    fill_outs_table(outs_of, rcp_gs);
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
    const bool gok = gains_finite<BPT>(gain);
    const int step = nblocks * tokens_per_block;
    int t = blk * tokens_per_block + sub;
    if (t < T) {
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const u32x4* p = &x[src[i] + static_cast<size_t>(t) * shard8];
            copy16_to_lds(p, &stage[2 * i][wbase]);
            copy16_to_lds(p + 1, &stage[2 * i + 1][wbase]);
        }
    }
    int par = 0;
    wait_copies();
    // block-uniform trip count (every wave reaches every barrier). Each
    // token's row has landed when its iteration starts: the wait for it
    // comes before the previous token's stores, so no iteration waits for
    // its predecessor's stores (the vector memory counter covers stores
    // too, and loads and stores may complete out of order against each
    // other, so the wait cannot single out the copies).
    for (int t0 = blk * tokens_per_block; t0 < T; t0 += step, t += step, par ^= 1) {
        // uniform in the wave; with one token per block always true here
        const bool tok_ok = TPT == kRowBlock || t < T;
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
        // (a wave with no token issued no copies: nothing to wait for)
        if (!tok_ok) continue;
        const float rinv = rms_inverse(ss, H, hf, inv_h, eps);
        const bool finite = gok && ss <= 3.40282347e38f && rinv <= 3.40282347e38f;
        uint2 codes[BPT];
        uint32_t sf[BPT];
#pragma unroll
        for (int i = 0; i < BPT; ++i)
            codes[i] = finite ? encode_block<true>(xw[i], gain[i], rinv, gs, outs_of, &sf[i])
                              : encode_block<false>(xw[i], gain[i], rinv, gs, outs_of, &sf[i]);
        // the next token's row has landed (its copies were issued before
        // this token's reduction); then this token's stores
        wait_copies();
#pragma unroll
        for (int i = 0; i < BPT; ++i) {
            const int b = tid + i * TPT;
            packed[static_cast<size_t>(t) * nblk + b] = codes[i];
            scales[static_cast<size_t>(t) * nblk + b] = static_cast<uint8_t>(sf[i]);
        }
    }
}

template <int BPT, int TPT>
__global__ __launch_bounds__(kRowBlock) void norm_quant_staged_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center, float eps,
    const float* __restrict__ global_scale, int T, int H, int shard8,
    uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    norm_quant_staged_body<BPT, TPT>(blockIdx.x, gridDim.x, x, norm_w, gain_center, eps, global_scale, T, H,
                                     shard8, packed, scales);
}

// The dispatch's place step and norm + quant in one launch: blocks below
// n_place place their tile of slots (place_body), the others run the
// staged norm + quant over the tokens. The two depend on nothing of each
// other, and the place step's few latency-bound blocks then run beside the
// bandwidth-bound norm + quant instead of before it, with no second stream
// to fork and join (TensorRT-LLM PR #21356, "Where they plug in": the
// expert input prepared beside the routing).
// NQ = kStagedNq: the staged norm + quant (one token per block, each block
// visiting several); NQ = kWave or kRowBlock: the one-pass form, for batches
// with fewer tokens than the launch has blocks (small batches); NQ = 0: the
// one-pass form for rows that fill neither (`tpt` threads a token, bounds
// checked).
constexpr int kStagedNq = -1;

template <int MODE, int BPT, int NQ = kStagedNq>
__global__ __launch_bounds__(kRowBlock) void place_norm_quant_kernel(
    int n_place, const int32_t* __restrict__ ids, int n, int E, int tile, int tiles,
    const int32_t* __restrict__ tile_hist, int32_t* __restrict__ counts, int32_t* __restrict__ offsets,
    int32_t* __restrict__ perm, int32_t* __restrict__ dest, const u32x4* __restrict__ x,
    const float* __restrict__ norm_w, float gain_center, float eps, const float* __restrict__ global_scale,
    int T, int H, int tpt, uint2* __restrict__ packed, uint8_t* __restrict__ scales) {
    static_assert(kDispBlock == kRowBlock, "one block size");
    extern __shared__ __attribute__((aligned(16))) int32_t place_lds[];
    if (static_cast<int>(blockIdx.x) < n_place)
        place_body<MODE>(blockIdx.x, place_lds, ids, n, E, tile, tiles, tile_hist, counts, offsets, perm, dest);
    else if constexpr (NQ == kStagedNq)
        norm_quant_staged_body<BPT, kRowBlock>(blockIdx.x - n_place, gridDim.x - n_place, x, norm_w, gain_center,
                                               eps, global_scale, T, H, H / 8, packed, scales);
    else
        norm_quant_body<BPT, NQ>(blockIdx.x - n_place, gridDim.x - n_place, x, norm_w, gain_center, eps,
                                 global_scale, T, H, H / 8, NQ == 0 ? tpt : NQ, packed, scales);
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

// Blocks per CU of the staged norm + quant (fewer than fit: each then visits
// more tokens, and fewer rows are in flight at once). At 8192 tokens of 8192
// after a read flush: 36.3 us at the 5 that fit, 36.3 at 4, 35.2-35.6 at 3,
// 34.6 at 2.
constexpr int kStagedPerCu = 3;

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
        const int fit = resident_blocks(norm_quant_staged_kernel<BPT, TPT>, kRowBlock, 0);
        const int cap_staged = device_cu_count() * (fit < kStagedPerCu ? fit : kStagedPerCu);
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

namespace moe {

int check_norm_quant(const uint16_t* x, const float* norm_w, float gain_center, float eps,
                     const float* global_scale, int T, int H, const uint8_t* packed, const uint8_t* scales) {
    if (T < 0 || H < 16 || H > MOE_MAX_HIDDEN || H % 16 != 0) return MOE_ERR_BAD_SHAPE;
    if (!std::isfinite(gain_center) || !std::isfinite(eps) || eps < 0.f) return MOE_ERR_BAD_ARG;
    if (T == 0) return MOE_OK;
    if (!x || !norm_w || !global_scale || !packed || !scales) return MOE_ERR_NULL_ARG;
    if (!all_aligned16(x, norm_w, packed, scales)) return MOE_ERR_ALIGN;
    return MOE_OK;
}

namespace {

template <int MODE, int BPT, int NQ = kStagedNq>
int launch_place_norm_quant(int grid, int n_place, size_t lds, const int32_t* topk_ids, int n, int E, int tile,
                            int tiles, int32_t* tile_counts, int32_t* counts, int32_t* offsets, int32_t* perm,
                            int32_t* dest, const uint16_t* x, const float* norm_w, float gain_center, float eps,
                            const float* global_scale, int T, int H, int tpt, uint8_t* packed, uint8_t* scales,
                            void* stream) {
    return launch(place_norm_quant_kernel<MODE, BPT, NQ>, dim3(grid), dim3(kRowBlock), lds, stream, n_place, topk_ids,
                  n, E, tile, tiles, static_cast<const int32_t*>(tile_counts), counts, offsets, perm, dest,
                  reinterpret_cast<const u32x4*>(x), norm_w, gain_center, eps, global_scale, T, H, tpt,
                  reinterpret_cast<uint2*>(packed), scales);
}

// Blocks of place_norm_quant_kernel<MODE, bpt, one_tpt> resident per CU.
template <int MODE>
int resident_place_norm_quant_one(int bpt, int one_tpt, size_t lds) {
    if (one_tpt == kWave) return resident_blocks(place_norm_quant_kernel<MODE, 1, kWave>, kRowBlock, lds);
    switch (bpt) {
        case 1: return resident_blocks(place_norm_quant_kernel<MODE, 1, kRowBlock>, kRowBlock, lds);
        case 2: return resident_blocks(place_norm_quant_kernel<MODE, 2, kRowBlock>, kRowBlock, lds);
        case 3: return resident_blocks(place_norm_quant_kernel<MODE, 3, kRowBlock>, kRowBlock, lds);
        default: return resident_blocks(place_norm_quant_kernel<MODE, 4, kRowBlock>, kRowBlock, lds);
    }
}

template <int MODE>
int resident_place_norm_quant(int bpt, size_t lds) {
    switch (bpt) {
        case 1: return resident_blocks(place_norm_quant_kernel<MODE, 1>, kRowBlock, lds);
        case 2: return resident_blocks(place_norm_quant_kernel<MODE, 2>, kRowBlock, lds);
        case 3: return resident_blocks(place_norm_quant_kernel<MODE, 3>, kRowBlock, lds);
        default: return resident_blocks(place_norm_quant_kernel<MODE, 4>, kRowBlock, lds);
    }
}

}  // namespace

int run_place_norm_quant(const int32_t* topk_ids, long long n, int E, int32_t* counts, int32_t* offsets,
                         int32_t* perm, int32_t* dest, int32_t* tile_counts, const uint16_t* x,
                         const float* norm_w, float gain_center, float eps, const float* global_scale, int T, int H,
                         uint8_t* packed, uint8_t* scales, void* stream) {
    const BlockGeom geo = block_geom(H);
    // the fused launch covers the staged norm + quant with one token per
    // block (H / 16 = 256 BPT) when every one of its blocks gets several
    // tokens, as the staged kernel is meant for
    const bool whole = geo.tpt == kRowBlock && H / 16 == geo.bpt * kRowBlock && geo.bpt <= 4;
    if (whole && n > 0 && T > 0) {
        const int mode = place_mode(n, E);
        const DispatchTiles d = dispatch_tiles(n);
        const int n_place = mode == kPlaceSingle ? 1 : d.tiles;
        const size_t lds = place_lds_bytes(mode, E);
        const int per_cu = mode == kPlaceSingle ? resident_place_norm_quant<kPlaceSingle>(geo.bpt, lds)
                           : mode == kPlaceFused ? resident_place_norm_quant<kPlaceFused>(geo.bpt, lds)
                                                 : resident_place_norm_quant<kPlaceScanned>(geo.bpt, lds);
        // every block resident at once
        const int grid = device_cu_count() * (per_cu < kStagedPerCu ? per_cu : kStagedPerCu);
        const int n_nq = grid - n_place;
        if (n_nq >= device_cu_count() && T > n_nq) {
            if (mode == kPlaceScanned) {
                const int rc = run_scan(tile_counts, n, E, counts, stream);
                if (rc) return rc;
            }
#define MOE_PNQ(M, B)                                                                                         \
    if (mode == M && geo.bpt == B)                                                                            \
        return launch_place_norm_quant<M, B>(grid, n_place, lds, topk_ids, static_cast<int>(n), E, d.tile, d.tiles, \
                                             tile_counts, counts, offsets, perm, dest, x, norm_w, gain_center, eps, \
                                             global_scale, T, H, kRowBlock, packed, scales, stream);
            MOE_PNQ(kPlaceSingle, 1) MOE_PNQ(kPlaceSingle, 2) MOE_PNQ(kPlaceSingle, 3) MOE_PNQ(kPlaceSingle, 4)
            MOE_PNQ(kPlaceFused, 1) MOE_PNQ(kPlaceFused, 2) MOE_PNQ(kPlaceFused, 3) MOE_PNQ(kPlaceFused, 4)
            MOE_PNQ(kPlaceScanned, 1) MOE_PNQ(kPlaceScanned, 2) MOE_PNQ(kPlaceScanned, 3) MOE_PNQ(kPlaceScanned, 4)
#undef MOE_PNQ
        }
    }
    // Otherwise (too few tokens for the staged form to pay, or rows of 64
    // blocks, one token per wave) the one-pass norm + quant shares the
    // launch, over as many blocks as its tokens need up to the GPU's resident
    // capacity; blocks beyond what is resident wait their turn, as nothing
    // waits on another block.
    const int one_tpt =
        (geo.tpt == kRowBlock || (geo.tpt == kWave && geo.bpt == 1)) && H / 16 == geo.bpt * geo.tpt && geo.bpt <= 4
            ? geo.tpt : 0;
    if (one_tpt && n > 0 && T > 0) {
        const int mode = place_mode(n, E);
        const DispatchTiles d = dispatch_tiles(n);
        const int n_place = mode == kPlaceSingle ? 1 : d.tiles;
        const size_t lds = place_lds_bytes(mode, E);
        const int per_cu = mode == kPlaceSingle ? resident_place_norm_quant_one<kPlaceSingle>(geo.bpt, one_tpt, lds)
                           : mode == kPlaceFused ? resident_place_norm_quant_one<kPlaceFused>(geo.bpt, one_tpt, lds)
                                                 : resident_place_norm_quant_one<kPlaceScanned>(geo.bpt, one_tpt, lds);
        const int needed = ceil_div(T, kRowBlock / one_tpt);
        const int room = device_cu_count() * per_cu - n_place;
        const int n_nq = min(needed, max(room, device_cu_count()));
        if (mode == kPlaceScanned) {
            const int rc = run_scan(tile_counts, n, E, counts, stream);
            if (rc) return rc;
        }
#define MOE_PNQ1(M, B, TP)                                                                                      \
    if (mode == M && geo.bpt == B && one_tpt == TP)                                                             \
        return launch_place_norm_quant<M, B, TP>(n_place + n_nq, n_place, lds, topk_ids, static_cast<int>(n), E,  \
                                                 d.tile, d.tiles, tile_counts, counts, offsets, perm, dest, x,    \
                                                 norm_w, gain_center, eps, global_scale, T, H, TP, packed,       \
                                                 scales, stream);
#define MOE_PNQ1_MODE(M) \
    MOE_PNQ1(M, 1, kWave) MOE_PNQ1(M, 1, kRowBlock) MOE_PNQ1(M, 2, kRowBlock) MOE_PNQ1(M, 3, kRowBlock) \
    MOE_PNQ1(M, 4, kRowBlock)
        MOE_PNQ1_MODE(kPlaceSingle) MOE_PNQ1_MODE(kPlaceFused) MOE_PNQ1_MODE(kPlaceScanned)
#undef MOE_PNQ1_MODE
#undef MOE_PNQ1
    }
    // Rows that fill neither a wave nor a block (fewer than 1024 or not a
    // multiple of 1024 wide), with every slot in one dispatch tile (small
    // batches): the generic one-pass form beside the single place block.
    if (n > 0 && T > 0 && geo.bpt <= 4 && place_mode(n, E) == kPlaceSingle) {
        const DispatchTiles d = dispatch_tiles(n);
        const size_t lds = place_lds_bytes(kPlaceSingle, E);
        const int needed = ceil_div(T, kRowBlock / geo.tpt);
        const int cap = device_cu_count() * 4;
        const int n_nq = needed < cap ? needed : cap;
#define MOE_PNQ0(B)                                                                                             \
    if (geo.bpt == B)                                                                                           \
        return launch_place_norm_quant<kPlaceSingle, B, 0>(1 + n_nq, 1, lds, topk_ids, static_cast<int>(n), E,   \
                                                           d.tile, d.tiles, tile_counts, counts, offsets, perm,  \
                                                           dest, x, norm_w, gain_center, eps, global_scale, T,   \
                                                           H, geo.tpt, packed, scales, stream);
        MOE_PNQ0(1) MOE_PNQ0(2) MOE_PNQ0(3) MOE_PNQ0(4)
#undef MOE_PNQ0
    }
    int rc = n > 0 ? run_place(topk_ids, n, E, counts, offsets, perm, dest, tile_counts, stream)
                   : run_dispatch_empty(counts, offsets, E, stream);
    if (rc) return rc;
    return moe_norm_quant_nvfp4(x, norm_w, gain_center, eps, global_scale, T, H, packed, scales, stream);
}

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
