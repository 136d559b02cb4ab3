// NVFP4 encoding helpers shared by the kernels that write NVFP4 (the
// pre-expert norm + quant and the expert FC1 epilogue): E2M1 codes, E4M3
// block-scale bytes, and the hardware FP4 conversion with unit scale.
//
// Format: vLLM API docs, vllm.models.muse_spark.nvidia.ops.prepare_trtllm_nvfp4
// (`_quantize_nvfp4_global_scale`: E2M1 codes rounded to nearest even and
// saturating, two per byte with the even element in the low nibble; E4M3
// scales per 16 elements).
#pragma once

#include "common.hpp"

namespace moe {

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

// Codes of a pair y0, y1 (or a packed BF16 pair) times `outs` into byte BYTE
// of `word`:
// q = y * outs with -0 turned into +0 (an FMA with a +0 addend rounds once,
// like the product), then v_cvt_scalef32_pk_fp4_f32 with unit scale, which
// rounds finite values to the nearest E2M1 value (ties to even code),
// saturates, and puts the first value in the low nibble.
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t word, float y0, float y1, float outs) {
    const float q0 = __builtin_fmaf(y0, outs, 0.0f);
    const float q1 = __builtin_fmaf(y1, outs, 0.0f);
    return __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(word, q0, q1, 1.0f, BYTE);
}
template <int BYTE>
__device__ __forceinline__ uint32_t fp4_pair(uint32_t word, uint32_t ypair, float outs) {
    return fp4_pair<BYTE>(word, bf16_lo(ypair), bf16_hi(ypair), outs);
}

// E4M3 byte of a block scale s >= 0 (or NaN): v_cvt_pk_fp8_f32 rounds to the
// nearest E4M3 value with ties to the even code, subnormals included, but
// turns magnitudes past 464 into NaN; clamping to 448 first gives the
// saturating conversion, and NaN keeps the NaN code 0x7F.
__device__ __forceinline__ uint32_t e4m3_scale_code(float s) {
    if (!(s == s)) return 0x7Fu;
    const float c = s > 448.f ? 448.f : s;
    return static_cast<uint32_t>(__builtin_amdgcn_cvt_pk_fp8_f32(c, 0.0f, 0, false)) & 0xFFu;
}

}  // namespace moe
