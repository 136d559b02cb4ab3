// moe_expert_fc1_nvfp4: the expert FC1 on NVFP4 input -- a gather grouped
// GEMM over the rows the dispatch groups per expert, Relu2, NVFP4 output.
//
// Method: TensorRT-LLM PR #21842 ("CuTe DSL act-fusion GEMMs: key the early
// accumulator release on the loop index"), description (the block-scaled
// gather grouped GEMM with a fused activation that is the NVFP4 MoE FC1; its
// Relu2 workload K 1024, N 2688, 512 experts, top-22; FP4 outputs with their
// scale factors); vLLM API docs, prepare_trtllm_nvfp4 (the NVFP4 format and
// the block quantiser); lmdeploy PR #4835, MoE gate v2 (rows grouped per
// expert in `perm` order, `offsets` per expert).
//
// Design (gfx950):
//  * CDNA4's block-scaled MFMA takes power-of-two (E8M0) scales per 32
//    elements, not NVFP4's E4M3 scales per 16 (its FP4 conversions with a
//    scale likewise use only the scale's exponent), so both operands are
//    dequantised exactly to BF16: the unit-scale FP4 -> FP32 conversion, an
//    FP32 multiply by the E4M3 scale (a code value has at most 2 significant
//    bits and a scale 4, so the product is exact), and a BF16 pack. The GEMM
//    then runs v_mfma_f32_32x32x16_bf16 with FP32 accumulation; the global
//    scales are applied once, as alpha = 1 / (gs_x * gs_w[e]) in the epilogue.
//  * Block tile 128 grouped rows x 128 output columns, four waves of 64 x 64.
//    K advances in stages of 64: the raw FP4 bytes and scale bytes of the
//    next stage are loaded into registers while the MFMAs of this stage run,
//    then dequantised into the other half of a double-buffered LDS tile
//    (rows of 128 bytes, 16-byte chunks XOR-swizzled by row).
//  * The tiles of each expert are found from `offsets` by a one-block kernel
//    (exclusive prefix of ceil(rows / 128) over experts); the GEMM grid is an
//    upper bound, blocks past the last tile leave at once. Blocks are
//    remapped so that each XCD walks a contiguous run of (column tile,
//    expert, row tile), keeping an expert's weight slice in its L2.
//  * Epilogue: alpha * acc, Relu2, staged in LDS as FP32, then each thread
//    quantises 16-column blocks with the pre-expert quantiser's FP32 steps
//    (hardware E4M3 and FP4 conversions, as there).
#include <cmath>

#include "launch.hpp"
#include "nvfp4.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFcBM = 128;              // grouped rows per block tile
constexpr int kFcBN = 128;              // output columns per block tile
constexpr int kFcKS = 64;               // K per stage
constexpr int kFcBlock = 256;
constexpr int kFcStageBytes = (kFcBM + kFcBN) * kFcKS * 2;      // A and B, BF16
constexpr int kFcYStride = kFcBN + 4;                             // floats per staged output row
constexpr size_t kFcLds = 2 * kFcStageBytes > kFcBM * kFcYStride * 4
                              ? 2 * kFcStageBytes : static_cast<size_t>(kFcBM) * kFcYStride * 4;

// tile_start[e] = sum over e' < e of ceil(rows(e') / kFcBM); tile_start[E] = total.
__global__ __launch_bounds__(kFcBlock) void fc1_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                             int32_t* __restrict__ tile_start) {
    __shared__ int32_t wsum[kFcBlock / kWave];
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
    const int chunk = (E + kFcBlock - 1) / kFcBlock;
    const int e0 = min(E, tid * chunk), e1 = min(E, e0 + chunk);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (max(offsets[e + 1] - offsets[e], 0) + kFcBM - 1) / kFcBM;
    int incl = local;
#pragma unroll
    for (int d = 1; d < kWave; d <<= 1) {
        const int o = __shfl_up(incl, d, kWave);
        if (lane >= d) incl += o;
    }
    if (lane == kWave - 1) wsum[wave] = incl;
    __syncthreads();
    int run = incl - local;
    for (int w = 0; w < wave; ++w) run += wsum[w];
    for (int e = e0; e < e1; ++e) {
        tile_start[e] = run;
        run += (max(offsets[e + 1] - offsets[e], 0) + kFcBM - 1) / kFcBM;
    }
    if (tid == kFcBlock - 1) tile_start[E] = run;
}

// Grouped positions past offsets[E] get zero codes and zero scales.
__global__ __launch_bounds__(256) void fc1_fill_kernel(const int32_t* __restrict__ offsets, int E, int P,
                                                       int N, u32x4* __restrict__ y_packed,
                                                       uint32_t* __restrict__ y_scales) {
    const int used = min(max(offsets[E], 0), P);
    const size_t pv = static_cast<size_t>(N) / 32;   // 16-byte vectors per packed row
    const size_t sv = static_cast<size_t>(N) / 64;   // 4-byte words per scale row
    const size_t n0 = static_cast<size_t>(used), n1 = static_cast<size_t>(P);
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    const size_t start = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x;
    for (size_t i = n0 * pv + start; i < n1 * pv; i += stride) y_packed[i] = u32x4{0u, 0u, 0u, 0u};
    for (size_t i = n0 * sv + start; i < n1 * sv; i += stride) y_scales[i] = 0u;
}

// 16 raw bytes (32 E2M1 codes) and their two scale bytes -> 16 packed BF16
// pairs: value = code value * scale, exact.
__device__ __forceinline__ void dequant32(const u32x4& raw, uint32_t sc2, uint32_t (&out)[16]) {
    const float s0 = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sc2 & 0xFFu), 0);
    const float s1 = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>((sc2 >> 8) & 0xFFu), 0);
    const uint32_t w[4] = {raw.x, raw.y, raw.z, raw.w};
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const float s = q < 2 ? s0 : s1;
#pragma unroll
        for (int b = 0; b < 4; ++b) {
            f32x2_t v;
            switch (b) {   // byte select must be a constant
                case 0: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 0); break;
                case 1: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 1); break;
                case 2: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 2); break;
                default: v = __builtin_amdgcn_cvt_scalef32_pk_f32_fp4(w[q], 1.0f, 3); break;
            }
            out[4 * q + b] = cvt_pk_bf16(v.x * s, v.y * s);
        }
    }
}

__device__ __forceinline__ int chunk_off(int row, int c) { return row * 128 + ((c ^ (row & 7)) << 4); }

__global__ __launch_bounds__(kFcBlock) __attribute__((amdgpu_waves_per_eu(2))) void fc1_gemm_kernel(
    const uint8_t* __restrict__ x_packed, const uint8_t* __restrict__ x_scales,
    const float* __restrict__ x_gs, const int32_t* __restrict__ perm, const int32_t* __restrict__ offsets,
    const int32_t* __restrict__ tile_start, int k, const uint8_t* __restrict__ w_packed,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs, const float* __restrict__ y_gs,
    int K, int N, int E, int n_pos, int m_upper, int per_xcd, uint8_t* __restrict__ y_packed,
    uint8_t* __restrict__ y_scales) {
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
    // XCD-contiguous logical tile index: (column tile, row tile over experts)
    const int logical = (blockIdx.x % 8) * per_xcd + blockIdx.x / 8;
    const int nt = logical / m_upper;
    const int mt = logical - nt * m_upper;
    if (nt >= N / kFcBN || mt >= tile_start[E]) return;
    // expert owning row tile mt: the last e with tile_start[e] <= mt
    int lo = 0, hi = E - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (tile_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int e = lo;
    const int row_end = min(offsets[e + 1], n_pos);
    const int m0 = offsets[e] + (mt - tile_start[e]) * kFcBM;
    const int n0 = nt * kFcBN;

    // this thread's load assignment: row r of both tiles, K half h of a stage
    const int r = tid >> 1, h = tid & 1;
    const int p = m0 + r;
    const int slot = p >= 0 && p < row_end ? perm[p] : -1;
    const bool a_ok = slot >= 0 && slot < n_pos;   // a slot outside [0, T k) reads nothing
    const int token = a_ok ? slot / k : 0;
    const size_t kb = static_cast<size_t>(K) / 2, ks = static_cast<size_t>(K) / 16;
    const uint8_t* xa = x_packed + static_cast<size_t>(token) * kb + h * 16;
    const uint8_t* xsa = x_scales + static_cast<size_t>(token) * ks + h * 2;
    const size_t wrow = static_cast<size_t>(e) * N + n0 + r;
    const uint8_t* wb = w_packed + wrow * kb + h * 16;
    const uint8_t* wsb = w_scales + wrow * ks + h * 2;

    u32x4 ra, rb;
    uint32_t sa, sb;
    auto load_raw = [&](int s) {
        const int kk = s * kFcKS;   // element offset of the stage
        ra = u32x4{0u, 0u, 0u, 0u};
        sa = 0u;
        if (a_ok) {
            ra = *reinterpret_cast<const u32x4*>(xa + kk / 2);
            sa = *reinterpret_cast<const uint16_t*>(xsa + kk / 16);
        }
        rb = *reinterpret_cast<const u32x4*>(wb + kk / 2);
        sb = *reinterpret_cast<const uint16_t*>(wsb + kk / 16);
    };
    auto store_stage = [&](int buf) {
        char* A = lds + buf * kFcStageBytes;
        char* B = A + kFcBM * kFcKS * 2;
        uint32_t d[16];
        dequant32(ra, sa, d);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4*>(A + chunk_off(r, 4 * h + c)) = u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
        dequant32(rb, sb, d);
#pragma unroll
        for (int c = 0; c < 4; ++c)
            *reinterpret_cast<u32x4*>(B + chunk_off(r, 4 * h + c)) = u32x4{d[4 * c], d[4 * c + 1], d[4 * c + 2], d[4 * c + 3]};
    };

    f32x16_t acc[2][2];
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int j = 0; j < 2; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int wm = wave >> 1, wn = wave & 1;
    const int frow = lane & 31, hc = lane >> 5;
    const int nst = K / kFcKS;

    load_raw(0);
    store_stage(0);
    __syncthreads();
    for (int s = 0; s < nst; ++s) {
        if (s + 1 < nst) load_raw(s + 1);
        const char* A = lds + (s & 1) * kFcStageBytes;
        const char* B = A + kFcBM * kFcKS * 2;
#pragma unroll
        for (int j = 0; j < kFcKS / 16; ++j) {
            bf16x8_t a[2], b[2];
#pragma unroll
            for (int i = 0; i < 2; ++i) {
                a[i] = *reinterpret_cast<const bf16x8_t*>(A + chunk_off(wm * 64 + i * 32 + frow, 2 * j + hc));
                b[i] = *reinterpret_cast<const bf16x8_t*>(B + chunk_off(wn * 64 + i * 32 + frow, 2 * j + hc));
            }
#pragma unroll
            for (int i = 0; i < 2; ++i)
#pragma unroll
                for (int jn = 0; jn < 2; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[i], b[jn], acc[i][jn], 0, 0, 0);
        }
        if (s + 1 < nst) store_stage((s + 1) & 1);
        __syncthreads();
    }

    // epilogue: y = Relu2(alpha * acc) staged in LDS (the stage buffers are
    // free: every wave passed the last barrier after its last MFMA reads)
    const float alpha = 1.0f / (*x_gs * w_gs[e]);
    float* Y = reinterpret_cast<float*>(lds);
    const int half = lane >> 5;
#pragma unroll
    for (int i = 0; i < 2; ++i)
#pragma unroll
        for (int jn = 0; jn < 2; ++jn) {
            const int col = wn * 64 + jn * 32 + (lane & 31);
#pragma unroll
            for (int q = 0; q < 16; ++q) {
                const int row = wm * 64 + i * 32 + 8 * (q >> 2) + 4 * half + (q & 3);
                const float v = alpha * acc[i][jn][q];
                const float rl = v > 0.f ? v : 0.f;
                Y[row * kFcYStride + col] = rl * rl;
            }
        }
    __syncthreads();

    const float gs = *y_gs;
    const float rcp_gs = 1.0f / gs;
    constexpr float kRcp6 = 1.0f / 6.0f;
    const size_t yrow_b = static_cast<size_t>(N) / 2, yrow_s = static_cast<size_t>(N) / 16;
#pragma unroll
    for (int u = 0; u < (kFcBM * kFcBN / 16) / kFcBlock; ++u) {
        const int q = tid + u * kFcBlock;
        const int row = q / (kFcBN / 16), cb = q - row * (kFcBN / 16);
        const int pr = m0 + row;
        const float4* src = reinterpret_cast<const float4*>(Y + row * kFcYStride + cb * 16);
        float y[16];
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const float4 f = src[v];
            y[4 * v] = f.x; y[4 * v + 1] = f.y; y[4 * v + 2] = f.z; y[4 * v + 3] = f.w;
        }
        float amax = 0.f;
#pragma unroll
        for (int v = 0; v < 16; ++v) amax = fmaxf(amax, y[v]);   // y >= 0
        const float s = gs * (amax * kRcp6);
        const uint32_t sf = e4m3_scale_code(s);
        const float sf_f = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sf), 0);
        const float d = sf_f * rcp_gs;
        const float outs = (sf_f != 0.f) ? 1.0f / d : 0.f;
        uint32_t w0 = 0, w1 = 0;
        if (amax < INFINITY && fabsf(outs) < INFINITY) {
            // y >= 0, so q = y * out is never -0; the hardware conversion with
            // unit scale rounds finite values to nearest even and saturates
            w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[0] * outs, y[1] * outs, 1.0f, 0);
            w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[2] * outs, y[3] * outs, 1.0f, 1);
            w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[4] * outs, y[5] * outs, 1.0f, 2);
            w0 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w0, y[6] * outs, y[7] * outs, 1.0f, 3);
            w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[8] * outs, y[9] * outs, 1.0f, 0);
            w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[10] * outs, y[11] * outs, 1.0f, 1);
            w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[12] * outs, y[13] * outs, 1.0f, 2);
            w1 = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w1, y[14] * outs, y[15] * outs, 1.0f, 3);
        } else {
#pragma unroll
            for (int v = 0; v < 8; ++v) {
                w0 |= e2m1_code(y[v] * outs) << (4 * v);
                w1 |= e2m1_code(y[8 + v] * outs) << (4 * v);
            }
        }
        if (pr >= 0 && pr < row_end) {
            *reinterpret_cast<uint2*>(y_packed + static_cast<size_t>(pr) * yrow_b + (n0 + cb * 16) / 2) = make_uint2(w0, w1);
            y_scales[static_cast<size_t>(pr) * yrow_s + n0 / 16 + cb] = static_cast<uint8_t>(sf);
        }
    }
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_expert_fc1_workspace_bytes(int E) {
    if (E < 1 || E > MOE_MAX_EXPERTS) return 0;
    return (static_cast<size_t>(E + 1) * sizeof(int32_t) + 255) / 256 * 256;
}

extern "C" int moe_expert_fc1_nvfp4(const uint8_t* x_packed, const uint8_t* x_scales,
                                    const float* x_global_scale, const int32_t* perm,
                                    const int32_t* offsets, int T, int k, const uint8_t* w_packed,
                                    const uint8_t* w_scales, const float* w_global_scale,
                                    const float* y_global_scale, int K, int N, int E,
                                    uint8_t* y_packed, uint8_t* y_scales, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    using namespace moe;
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_BAD_SHAPE;
    if (K < kFcKS || K > MOE_MAX_HIDDEN || K % kFcKS != 0 || N < kFcBN || N % kFcBN != 0 ||
        N > 8 * MOE_MAX_HIDDEN)
        return MOE_ERR_BAD_SHAPE;
    const long long P = static_cast<long long>(T) * k;
    if (P >= (1ll << 31)) return MOE_ERR_BAD_SHAPE;
    if (T == 0) return MOE_OK;
    if (!x_packed || !x_scales || !x_global_scale || !perm || !offsets || !w_packed || !w_scales ||
        !w_global_scale || !y_global_scale || !y_packed || !y_scales)
        return MOE_ERR_NULL_ARG;
    if (!all_aligned16(x_packed, w_packed, y_packed, y_scales)) return MOE_ERR_ALIGN;
    if ((reinterpret_cast<uintptr_t>(x_scales) | reinterpret_cast<uintptr_t>(w_scales)) & 3u)
        return MOE_ERR_ALIGN;
    const size_t need = moe_expert_fc1_workspace_bytes(E);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    int32_t* tile_start = static_cast<int32_t*>(workspace);

    int rc = launch(fc1_tiles_kernel, dim3(1), dim3(kFcBlock), 0, stream, offsets, E, tile_start);
    if (rc) return rc;
    const int cap = device_cu_count() * 8;
    const long long fill_vec = P * (N / 32);
    const int gf = static_cast<int>(fill_vec / 256 + 1 < cap ? fill_vec / 256 + 1 : cap);
    rc = launch(fc1_fill_kernel, dim3(gf), dim3(256), 0, stream, offsets, E, static_cast<int>(P), N,
                reinterpret_cast<u32x4*>(y_packed), reinterpret_cast<uint32_t*>(y_scales));
    if (rc) return rc;
    // row tiles over experts: at most ceil(P / BM) + E
    const long long m_upper = (P + kFcBM - 1) / kFcBM + E;
    const long long tiles = m_upper * (N / kFcBN);
    const long long per_xcd = (tiles + 7) / 8;
    if (per_xcd * 8 >= (1ll << 31)) return MOE_ERR_BAD_SHAPE;
    return launch(fc1_gemm_kernel, dim3(static_cast<unsigned>(per_xcd * 8)), dim3(kFcBlock), kFcLds,
                  stream, x_packed, x_scales, x_global_scale, perm, offsets,
                  static_cast<const int32_t*>(tile_start), k, w_packed, w_scales, w_global_scale,
                  y_global_scale, K, N, E, static_cast<int>(P), static_cast<int>(m_upper),
                  static_cast<int>(per_xcd), y_packed, y_scales);
}
