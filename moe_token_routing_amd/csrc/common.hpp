// Shared device helpers of the gfx950 kernels (wave64, CDNA4).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe_routing.h"

namespace moe {

constexpr int kWave = 64;

// 16-byte vector of four 32-bit words (a native vector type, so the
// non-temporal load/store builtins accept it).
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

__device__ __forceinline__ u32x4 load_nt(const u32x4* p) { return __builtin_nontemporal_load(p); }
__device__ __forceinline__ void store_nt(u32x4 v, u32x4* p) { __builtin_nontemporal_store(v, p); }

// ---- BF16 bit patterns ------------------------------------------------------

__device__ __forceinline__ float bf16_lo(uint32_t packed) {   // element 2m of a packed pair
    return __uint_as_float(packed << 16);
}
__device__ __forceinline__ float bf16_hi(uint32_t packed) {   // element 2m+1
    return __uint_as_float(packed & 0xFFFF0000u);
}

typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

// x0^2 + x1^2 + acc for a packed BF16 pair (v_dot2_f32_bf16; the products
// are exact in FP32).
__device__ __forceinline__ float dot2_sq(uint32_t packed, float acc) {
    const bf16x2_t b = __builtin_bit_cast(bf16x2_t, packed);
    return __builtin_amdgcn_fdot2_f32_bf16(b, b, acc, false);
}

// Two FP32 values -> packed BF16 pair, round to nearest even (v_cvt_pk_bf16_f32).
__device__ __forceinline__ uint32_t cvt_pk_bf16(float lo, float hi) {
    const f32x2_t v = {lo, hi};
    return __builtin_bit_cast(uint32_t, __builtin_convertvector(v, bf16x2_t));
}

typedef uint16_t u16x2_t __attribute__((ext_vector_type(2)));

// Lane-wise unsigned maximum of two packed 16-bit pairs (v_pk_max_u16).
__device__ __forceinline__ uint32_t packed_max_u16(uint32_t a, uint32_t b) {
    const u16x2_t r = __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a), __builtin_bit_cast(u16x2_t, b));
    return __builtin_bit_cast(uint32_t, r);
}

// FP32 -> BF16, round to nearest even; NaN stays a quiet NaN with its sign.
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return (u >> 16) | 0x40u;
    u += 0x7FFFu + ((u >> 16) & 1u);
    return u >> 16;
}
__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
    return f32_to_bf16_rne(lo) | (f32_to_bf16_rne(hi) << 16);
}

// ---- wave reductions (wave64) ---------------------------------------------

// Sum over the wave as a butterfly: v += v[lane ^ d] for d = 32, 16, 8, 4, 2,
// 1. Partners add the same two values, so every lane ends with the same sum
// and the order of additions is fixed. The exchanges use no LDS addresses:
// d = 32 and 16 swap row halves between two copies of v (v_permlane32_swap,
// v_permlane16_swap: each copy then holds one operand of every lane's
// addition), d = 8 rotates a 16-lane row by 8 and d = 2, 1 permute quads
// (DPP), and d = 4 is a ds_swizzle with xor mask 4.
__device__ __forceinline__ float wave_sum(float v) {
    uint32_t u = __float_as_uint(v);
    const auto s32 = __builtin_amdgcn_permlane32_swap(u, u, false, false);
    v = __uint_as_float(s32[0]) + __uint_as_float(s32[1]);
    u = __float_as_uint(v);
    const auto s16 = __builtin_amdgcn_permlane16_swap(u, u, false, false);
    v = __uint_as_float(s16[0]) + __uint_as_float(s16[1]);
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x128, 0xF, 0xF, false));   // row_ror:8
    v += __int_as_float(__builtin_amdgcn_ds_swizzle(__float_as_int(v), 0x101F));   // lane ^ 4 (32-lane groups)
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));    // quad [2,3,0,1]
    v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));    // quad [1,0,3,2]
    return v;
}

// Sum over aligned groups of `width` lanes (width a power of two <= 64).
__device__ __forceinline__ float group_sum(float v, int width) {
    for (int off = width >> 1; off >= 1; off >>= 1) v += __shfl_xor(v, off, kWave);
    return v;
}

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) {
        uint64_t o = __shfl_xor(v, off, kWave);
        v = o > v ? o : v;
    }
    return v;
}

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }

__device__ __forceinline__ uint64_t lanemask_lt() {
    const int lane = __lane_id();
    return lane == 0 ? 0ull : (~0ull >> (64 - lane));
}

inline int ceil_div(long long a, long long b) { return (int)((a + b - 1) / b); }

// NULL counts as aligned; NULL checks are separate.
inline bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
template <typename... P>
inline bool all_aligned16(const P*... p) { return (aligned16(p) && ...); }

inline int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

}  // namespace moe
