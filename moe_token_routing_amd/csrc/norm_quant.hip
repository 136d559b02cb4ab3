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
// registers; its sum of squares is reduced across the token's threads; each
// 16-element block is two neighbouring 8-element vectors held by adjacent
// lanes, so the block maximum is one lane swap. Codes leave as one 32-bit
// store per 8 elements, scales as one byte per block.
#include <cmath>

#include "launch.hpp"
#include "rows.hpp"

namespace moe {
namespace {

__device__ __forceinline__ float round_to_bf16(float f) {
    return __uint_as_float(f32_to_bf16_rne(f) << 16);
}

// E4M3 (no infinities, max 448): nearest value, ties to even code, magnitudes
// above 448 saturate, NaN -> 0x7F. Works on |s| and puts the sign in bit 7.
__device__ __forceinline__ uint32_t e4m3_satfinite(float s) {
    if (!(s == s)) return 0x7Fu;
    const uint32_t sign = (__float_as_uint(s) >> 24) & 0x80u;
    const float a = fabsf(s);
    uint32_t code;
    if (a >= 448.f) {
        code = 0x7Eu;
    } else if (a < 0x1p-6f) {
        // subnormal range: multiples of 2^-9; 8 * 2^-9 = 2^-6 is code 0x08
        code = static_cast<uint32_t>(rintf(a * 512.f));
    } else {
        const int e = static_cast<int>((__float_as_uint(a) >> 23) & 0xFFu) - 127;   // -6..8
        const float m = ldexpf(a, -e);                                            // [1, 2)
        code = static_cast<uint32_t>((e + 7) << 3) + static_cast<uint32_t>(rintf((m - 1.f) * 8.f));
    }
    return code | sign;
}

__device__ __forceinline__ float e4m3_value(uint32_t c) {
    const uint32_t mag = c & 0x7Fu;
    float v;
    if (mag == 0x7Fu) {
        v = __uint_as_float(0x7FC00000u);
    } else {
        const uint32_t e = mag >> 3, m = mag & 7u;
        v = e == 0 ? static_cast<float>(m) * 0x1p-9f
                   : ldexpf(static_cast<float>(8u + m), static_cast<int>(e) - 10);
    }
    return (c & 0x80u) ? -v : v;
}

// FP4 E2M1 code: magnitude rounded to the nearest of {0,.5,1,1.5,2,3,4,6}
// with ties to the even code, saturating; bit 3 when q < 0; NaN -> 0.
// Within [0,2) the grid step is 1/2, within [2,4) it is 1, from 4 it is 2, and
// in each range the code parity equals the parity of the rounded step count.
__device__ __forceinline__ uint32_t e2m1_code(float q) {
    const float a = fabsf(q);
    uint32_t c;
    if (!(a == a)) {
        c = 0u;
    } else if (a < 2.f) {
        c = static_cast<uint32_t>(rintf(a * 2.f));
    } else if (a < 4.f) {
        c = 4u + static_cast<uint32_t>(rintf(a - 2.f));
    } else {
        c = rintf((a - 4.f) * 0.5f) >= 1.f ? 7u : 6u;
    }
    return c | (q < 0.f ? 8u : 0u);
}

// Codes of a packed BF16 pair y times `outs` into byte BYTE of `word`:
// q = y * outs with -0 turned into +0 (an FMA with a +0 addend rounds once,
// like the product), then v_cvt_scalef32_pk_fp4_f32 with unit scale, which
// rounds finite values to the nearest E2M1 value (ties to even code),
// saturates, and puts the first value in the low nibble.
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t word, uint32_t ypair, float outs) {
    const float q0 = __builtin_fmaf(bf16_lo(ypair), outs, 0.0f);
    const float q1 = __builtin_fmaf(bf16_hi(ypair), outs, 0.0f);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, BYTE);
}

template <int VPT>
__global__ __launch_bounds__(kRowBlock) void norm_quant_kernel(
    const u32x4* __restrict__ x, const float* __restrict__ norm_w, float gain_center, float eps,
    const float* __restrict__ global_scale, int T, int H, int shard8, int tpt,
    uint32_t* __restrict__ packed, uint8_t* __restrict__ scales) {
    __shared__ float red[kRowBlock / kWave];
    const int nvec = H >> 3;
    const int tokens_per_block = kRowBlock / tpt;
    const int sub = threadIdx.x / tpt;
    const int tid = threadIdx.x - sub * tpt;
    const float hf = static_cast<float>(H);
    const float gs = *global_scale;
    const float rcp_gs = 1.0f / gs;
    constexpr float kRcp6 = 1.0f / 6.0f;

    float gain[VPT][8];
    // vector v (logical columns [8v, 8v+8)) of token t sits at
    // src[i] + t * shard8 (16-byte units), rank block v / shard8
    size_t src[VPT];
#pragma unroll
    for (int i = 0; i < VPT; ++i) {
        const int v = tid + i * tpt;
        const int rb = v / shard8;
        src[i] = static_cast<size_t>(rb) * T * shard8 + (v - rb * shard8);
#pragma unroll
        for (int e = 0; e < 8; ++e) gain[i][e] = 0.f;
        if (v < nvec) {
            const float4 a = reinterpret_cast<const float4*>(norm_w)[2 * v];
            const float4 b = reinterpret_cast<const float4*>(norm_w)[2 * v + 1];
            gain[i][0] = gain_center + a.x; gain[i][1] = gain_center + a.y;
            gain[i][2] = gain_center + a.z; gain[i][3] = gain_center + a.w;
            gain[i][4] = gain_center + b.x; gain[i][5] = gain_center + b.y;
            gain[i][6] = gain_center + b.z; gain[i][7] = gain_center + b.w;
        }
    }

    for (int t0 = blockIdx.x * tokens_per_block; t0 < T; t0 += gridDim.x * tokens_per_block) {
        const int t = t0 + sub;
        const bool tok_ok = t < T;
        u32x4 xv[VPT];
        float ss[1] = {0.f};
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + i * tpt;
            xv[i] = u32x4{0u, 0u, 0u, 0u};
            if (tok_ok && v < nvec) xv[i] = load_nt(&x[src[i] + static_cast<size_t>(t) * shard8]);
        }
#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            ss[0] = dot2_sq(xv[i].x, ss[0]);
            ss[0] = dot2_sq(xv[i].y, ss[0]);
            ss[0] = dot2_sq(xv[i].z, ss[0]);
            ss[0] = dot2_sq(xv[i].w, ss[0]);
        }
        token_sum(ss, tpt, red);
        const float rinv = 1.0f / sqrtf(ss[0] / hf + eps);

#pragma unroll
        for (int i = 0; i < VPT; ++i) {
            const int v = tid + i * tpt;
            const uint32_t w4[4] = {xv[i].x, xv[i].y, xv[i].z, xv[i].w};
            // normalised pairs, rounded once to BF16 (packed)
            uint32_t yp[4];
#pragma unroll
            for (int q = 0; q < 4; ++q)
                yp[q] = cvt_pk_bf16((bf16_lo(w4[q]) * gain[i][2 * q]) * rinv,
                                    (bf16_hi(w4[q]) * gain[i][2 * q + 1]) * rinv);
            // block maximum of |y|: the magnitude bits of non-negative BF16
            // values order like integers, and a NaN magnitude exceeds inf.
            const uint32_t m01 = packed_max_u16(yp[0] & 0x7FFF7FFFu, yp[1] & 0x7FFF7FFFu);
            const uint32_t m23 = packed_max_u16(yp[2] & 0x7FFF7FFFu, yp[3] & 0x7FFF7FFFu);
            const uint32_t m = packed_max_u16(m01, m23);
            uint32_t mbits = max(m & 0xFFFFu, m >> 16);
            mbits = max(mbits, static_cast<uint32_t>(__shfl_xor(static_cast<int>(mbits), 1, kWave)));
            const float bmax = __uint_as_float(mbits << 16);
            const float tq = bmax * kRcp6;
            const float s = gs * tq;
            const uint32_t sf = e4m3_satfinite(s);
            const float sf_f = e4m3_value(sf);
            const float d = sf_f * rcp_gs;
            const float outs = (sf_f != 0.f) ? 1.0f / d : 0.f;
            uint32_t word = 0;
            if (mbits < 0x7F80u && fabsf(outs) < INFINITY) {
                // q = y * out with -0 turned into +0 (fma with a +0 addend, one
                // rounding); the hardware E2M1 conversion with unit scale rounds
                // finite values to nearest even and saturates.
                word = fp4_pair<0>(word, yp[0], outs);
                word = fp4_pair<1>(word, yp[1], outs);
                word = fp4_pair<2>(word, yp[2], outs);
                word = fp4_pair<3>(word, yp[3], outs);
            } else {
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    word |= e2m1_code(bf16_lo(yp[q]) * outs) << (8 * q);
                    word |= e2m1_code(bf16_hi(yp[q]) * outs) << (8 * q + 4);
                }
            }
            if (tok_ok && v < nvec) {
                packed[static_cast<size_t>(t) * nvec + v] = word;
                if ((v & 1) == 0) scales[static_cast<size_t>(t) * (nvec >> 1) + (v >> 1)] = static_cast<uint8_t>(sf);
            }
        }
    }
}

template <int VPT>
int launch_norm_quant(const uint16_t* x, const float* norm_w, float gain_center, float eps,
                      const float* global_scale, int T, int H, int shard, const RowGeom& geo,
                      uint8_t* packed, uint8_t* scales, void* stream) {
    const int tokens_per_block = kRowBlock / geo.tpt;
    const int needed = ceil_div(T, tokens_per_block);
    const int cap = device_cu_count() * 8;
    const int grid = needed < cap ? needed : cap;
    return launch(norm_quant_kernel<VPT>, dim3(grid), dim3(kRowBlock), 0, stream,
                  reinterpret_cast<const u32x4*>(x), norm_w, gain_center, eps, global_scale, T, H,
                  shard / 8, geo.tpt, reinterpret_cast<uint32_t*>(packed), scales);
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
    const RowGeom geo = row_geom(H);
    int vpt = 1;
    while (vpt < geo.vpt) vpt <<= 1;
    switch (vpt) {
        case 1: return launch_norm_quant<1>(x, norm_w, gain_center, eps, global_scale, T, H, shard, geo, packed, scales, stream);
        case 2: return launch_norm_quant<2>(x, norm_w, gain_center, eps, global_scale, T, H, shard, geo, packed, scales, stream);
        case 4: return launch_norm_quant<4>(x, norm_w, gain_center, eps, global_scale, T, H, shard, geo, packed, scales, stream);
        case 8: return launch_norm_quant<8>(x, norm_w, gain_center, eps, global_scale, T, H, shard, geo, packed, scales, stream);
        default: return MOE_ERR_BAD_SHAPE;
    }
}

extern "C" int moe_norm_quant_nvfp4(const uint16_t* x, const float* norm_w, float gain_center,
                                    float eps, const float* global_scale, int T, int H,
                                    uint8_t* packed, uint8_t* scales, void* stream) {
    if (H < 16 || H % 16 != 0) return MOE_ERR_BAD_SHAPE;
    return moe_norm_quant_nvfp4_rank_block(x, H, norm_w, gain_center, eps, global_scale, T, H, packed,
                                           scales, stream);
}
