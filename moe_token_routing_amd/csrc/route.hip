// moe_route: router projection, sigmoid + bias selection, sorted top-k with
// lowest-id ties, renormalised weights, per-token validity mask.
//
// Method: TensorRT-LLM PR #21356 ("Add the Muse Spark Open decoder fast
// paths"), description, Triton kernels "Router projection" (FP32 weights and
// accumulation, scale folded in, tensor cores from 16 tokens) and "Routing";
// section "Not in this PR" (a BF16x3 router); TensorRT-LLM PR #21042 ("Add
// the Muse Spark Open model"), "MoE" (FP32 router); lmdeploy PR #4835, MoE
// gate v2 (required validity mask; aux-loss-free gate: bias for selection).
//
// Design (gfx950):
//  * The projection is a dense contraction, so it runs on MFMA. FP32 weights
//    are split exactly into three BF16 planes, W = W0 + W1 + W2 (each plane
//    holds the next 8 significant bits of what the previous ones missed; for
//    |W| >= 2^-100 the sum is exact). A BF16 input times a BF16 plane is exact
//    in FP32, so the three MFMA products h*W0 + h*W1 + h*W2 accumulate exact
//    products of the FP32 weights in FP32 (v_mfma_f32_32x32x16_bf16). An FP32
//    input is split the same way and the six products with plane-index sum
//    <= 2 are accumulated (the three dropped ones are below 2^-23 of |h*W|).
//  * Block tile 64 tokens x 64 experts, four waves of 32x32, K staged through
//    LDS in 32-wide chunks; split-K over a third grid dimension when the
//    tile grid alone cannot fill the GPU. Partial sums go to the workspace.
//  * The select kernel (one wave per token) adds the split-K partials in a
//    fixed order, applies the scale, evaluates the sigmoid in FP64 and rounds
//    it once, adds the bias in FP32 and picks the top k with k wave-wide
//    maximum reductions over 64-bit keys (ordered key bits, then inverted
//    expert id, so an exact tie goes to the lower id).
#include <cmath>

#include "launch.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kBM = 64;     // tokens per block tile
constexpr int kBN = 64;     // experts per block tile
constexpr int kKC = 32;     // K per LDS stage
constexpr int kLdsRow = kKC + 8;   // padded row (bf16 elements)
constexpr int kGemmBlock = 256;
constexpr int kTargetBlocks = 512;

// ---------------------------------------------------------------- split ----

// x (FP32) -> three BF16 planes whose sum is x.
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ x, size_t n,
                                                     uint16_t* __restrict__ planes) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        const float v = x[i];
        const uint32_t p0 = f32_to_bf16_rne(v);
        const float r1 = v - __uint_as_float(p0 << 16);
        const uint32_t p1 = f32_to_bf16_rne(r1);
        const float r2 = r1 - __uint_as_float(p1 << 16);
        const uint32_t p2 = f32_to_bf16_rne(r2);
        planes[i] = static_cast<uint16_t>(p0);
        planes[n + i] = static_cast<uint16_t>(p1);
        planes[2 * n + i] = static_cast<uint16_t>(p2);
    }
}

// ----------------------------------------------------------------- gemm ----

// Loads a [rows x kKC] tile (row stride ld elements) of a BF16 matrix into LDS
// rows [0, rows_max) with zero fill outside [0, nrows) x [k0, k1).
__device__ __forceinline__ void stage_tile(const uint16_t* __restrict__ src, int ld, int row0,
                                           int nrows, int k0, int k1, uint16_t* dst, int tid) {
    // kBM rows x (kKC / 8) vectors of 16 bytes = 256 vectors: one per thread.
    const int r = tid >> 2;
    const int c = (tid & 3) * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    const int row = row0 + r;
    const int k = k0 + c;
    if (row < nrows && k < k1) v = *reinterpret_cast<const uint4*>(src + static_cast<size_t>(row) * ld + k);
    *reinterpret_cast<uint4*>(dst + r * kLdsRow + c) = v;
}

__device__ __forceinline__ bf16x8_t lds_frag(const uint16_t* base, int row, int k) {
    const uint4 v = *reinterpret_cast<const uint4*>(base + row * kLdsRow + k);
    bf16x8_t f;
    __builtin_memcpy(&f, &v, 16);
    return f;
}

// NA: number of input planes (1 = BF16 input, 3 = split FP32 input).
template <int NA>
__global__ __launch_bounds__(kGemmBlock) void proj_kernel(
    const uint16_t* __restrict__ a_planes, const uint16_t* __restrict__ w_planes, int T, int H,
    int E, int kslice, float* __restrict__ partials) {
    __shared__ __attribute__((aligned(16))) uint16_t As[NA][kBM * kLdsRow];
    __shared__ __attribute__((aligned(16))) uint16_t Bs[3][kBN * kLdsRow];

    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int wm = (wave >> 1) * 32;   // wave's token offset in the tile
    const int wn = (wave & 1) * 32;    // wave's expert offset in the tile
    const int n0 = blockIdx.x * kBN;
    const int m0 = blockIdx.y * kBM;
    const int split = blockIdx.z;
    const int kbeg = split * kslice;
    const int kend = min(H, kbeg + kslice);
    const size_t a_plane = static_cast<size_t>(T) * H;
    const size_t w_plane = static_cast<size_t>(E) * H;

    f32x16_t acc;
#pragma unroll
    for (int i = 0; i < 16; ++i) acc[i] = 0.f;

    const int frow = lane & 31;          // fragment row (token or expert)
    const int fk = (lane >> 5) * 8;      // fragment k offset within a 16-wide step

    for (int k0 = kbeg; k0 < kend; k0 += kKC) {
#pragma unroll
        for (int p = 0; p < NA; ++p) stage_tile(a_planes + p * a_plane, H, m0, T, k0, kend, As[p], tid);
#pragma unroll
        for (int p = 0; p < 3; ++p) stage_tile(w_planes + p * w_plane, H, n0, E, k0, kend, Bs[p], tid);
        __syncthreads();
#pragma unroll
        for (int ks = 0; ks < kKC; ks += 16) {
            bf16x8_t a[NA], b[3];
#pragma unroll
            for (int p = 0; p < NA; ++p) a[p] = lds_frag(As[p], wm + frow, ks + fk);
#pragma unroll
            for (int p = 0; p < 3; ++p) b[p] = lds_frag(Bs[p], wn + frow, ks + fk);
            if constexpr (NA == 1) {
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], acc, 0, 0, 0);
            } else {
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[0], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[0], b[2], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[1], b[1], acc, 0, 0, 0);
                acc = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[2], b[0], acc, 0, 0, 0);
            }
        }
        __syncthreads();
    }

    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8*(i/4) + 4*(lane/32) + (i%4) for i = 0..15.
    float* out = partials + static_cast<size_t>(split) * T * E;
    const int col = n0 + wn + (lane & 31);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int row = m0 + wm + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
        if (row < T && col < E) out[static_cast<size_t>(row) * E + col] = acc[i];
    }
}

// --------------------------------------------------------------- select ----

// Monotone map of FP32 keys to unsigned integers; -0 counts as +0 and NaN
// ranks below every number.
__device__ __forceinline__ uint32_t ordered_key(float key) {
    uint32_t u = __float_as_uint(key);
    if (u == 0x80000000u) u = 0u;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

__device__ __forceinline__ float sigmoid_rn(float l) {
    return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
}

constexpr int kSelectBlock = 256;   // four tokens per block, one per wave

// EPL: experts per lane (E <= 64 * EPL). Expert e lives in lane e % 64, slot e / 64.
template <int EPL>
__global__ __launch_bounds__(kSelectBlock) void select_kernel(
    const float* __restrict__ partials, int nsplit, float scale, int logits_in,
    const float* __restrict__ bias, const uint8_t* __restrict__ token_mask, int T, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
    const int lane = __lane_id();
    const int t = blockIdx.x * (kSelectBlock / kWave) + threadIdx.x / kWave;
    if (t >= T) return;   // whole wave leaves together
    const size_t plane = static_cast<size_t>(T) * E;

    float lg[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        lg[i] = 0.f;
        if (e < E) {
            const size_t idx = static_cast<size_t>(t) * E + e;
            if (logits_in) {
                lg[i] = logits[idx];
            } else {
                float s = partials[idx];
                for (int p = 1; p < nsplit; ++p) s += partials[p * plane + idx];
                lg[i] = s * scale;
                logits[idx] = lg[i];
            }
        }
    }
    const size_t obase = static_cast<size_t>(t) * k;
    if (token_mask[t] == 0) {
        for (int j = lane; j < k; j += kWave) {
            topk_ids[obase + j] = -1;
            topk_w[obase + j] = 0.f;
        }
        return;
    }

    uint64_t cand[EPL];
    float sig[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const int e = lane + kWave * i;
        cand[i] = 0ull;
        sig[i] = 0.f;
        if (e < E) {
            sig[i] = sigmoid_rn(lg[i]);
            const float key = sig[i] + bias[e];
            cand[i] = (static_cast<uint64_t>(ordered_key(key)) << 32) | (0xFFFFFFFFu - static_cast<uint32_t>(e));
        }
    }

    int my_id = -1;
    float my_s = 0.f;
    for (int j = 0; j < k; ++j) {
        uint64_t best = 0ull;
        float best_s = 0.f;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            if (cand[i] > best) {
                best = cand[i];
                best_s = sig[i];
            }
        }
        const uint64_t win = wave_max_u64(best);
        const int id = static_cast<int>(0xFFFFFFFFu - static_cast<uint32_t>(win));
        const float s_win = __shfl(best_s, id & (kWave - 1), kWave);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if (cand[i] == win) cand[i] = 0ull;
        if (lane == j) {
            my_id = id;
            my_s = s_win;
        }
    }
    // FP32 running sum of the picked sigmoids in pick order (every lane the same).
    float total = 0.f;
    for (int j = 0; j < k; ++j) total += __shfl(my_s, j, kWave);
    if (lane < k) {
        topk_ids[obase + lane] = my_id;
        topk_w[obase + lane] = my_s / total;
    }
}

struct RoutePlan {
    int tiles_m, tiles_n, nsplit, kslice;
    size_t w_planes_bytes, a_planes_bytes, partial_bytes;
};

inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }

inline RoutePlan plan_route(int T, int H, int E, int hidden_dtype) {
    RoutePlan p;
    p.tiles_m = ceil_div(T, kBM);
    p.tiles_n = ceil_div(E, kBN);
    const int tiles = p.tiles_m * p.tiles_n;
    const int chunks = ceil_div(H, kKC);
    int ns = ceil_div(kTargetBlocks, tiles > 0 ? tiles : 1);
    if (ns > chunks) ns = chunks;
    if (ns < 1) ns = 1;
    const int per = ceil_div(chunks, ns);   // chunks per split
    p.kslice = per * kKC;
    p.nsplit = ceil_div(H, p.kslice);
    p.w_planes_bytes = round256(static_cast<size_t>(3) * E * H * sizeof(uint16_t));
    p.a_planes_bytes = hidden_dtype == MOE_DTYPE_F32 ? round256(static_cast<size_t>(3) * T * H * sizeof(uint16_t)) : 0;
    p.partial_bytes = round256(static_cast<size_t>(p.nsplit) * T * E * sizeof(float));
    return p;
}

template <int EPL>
int launch_select(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
                  const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
                  void* stream) {
    const int grid = ceil_div(T, kSelectBlock / kWave);
    return launch(select_kernel<EPL>, dim3(grid), dim3(kSelectBlock), 0, stream, partials, nsplit,
                  scale, logits_in, bias, mask, T, E, k, logits, ids, w);
}

int run_select(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
               const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
               void* stream) {
    const int epl = ceil_div(E, kWave);
#define MOE_SELECT(N) \
    if (epl <= N) return launch_select<N>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, stream);
    MOE_SELECT(1) MOE_SELECT(2) MOE_SELECT(4) MOE_SELECT(8) MOE_SELECT(16) MOE_SELECT(24)
    MOE_SELECT(32) MOE_SELECT(40) MOE_SELECT(48) MOE_SELECT(64)
#undef MOE_SELECT
    return MOE_ERR_BAD_SHAPE;
}

}  // namespace
}  // namespace moe

extern "C" size_t moe_route_workspace_bytes(int T, int H, int E, int k, int hidden_dtype, int logits_in) {
    using namespace moe;
    if (T <= 0 || H <= 0 || E <= 0 || k <= 0 || logits_in) return 0;
    if (hidden_dtype != MOE_DTYPE_F32 && hidden_dtype != MOE_DTYPE_BF16) return 0;
    const RoutePlan p = plan_route(T, H, E, hidden_dtype);
    return p.w_planes_bytes + p.a_planes_bytes + p.partial_bytes;
}

extern "C" int moe_route(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                         const uint8_t* token_mask, float scale, int T, int H, int E, int k,
                         float* logits, int32_t* topk_ids, float* topk_w, void* workspace,
                         size_t workspace_bytes, void* stream) {
    using namespace moe;
    const bool logits_in = hidden == nullptr;
    if (!logits_in && hidden_dtype != MOE_DTYPE_F32 && hidden_dtype != MOE_DTYPE_BF16)
        return MOE_ERR_BAD_DTYPE;
    if (T < 0 || H < 1 || H > MOE_MAX_HIDDEN || H % 16 != 0 || E < 1 || E > MOE_MAX_EXPERTS ||
        k < 1 || k > E || k > MOE_MAX_TOPK)
        return MOE_ERR_BAD_SHAPE;
    if (static_cast<long long>(T) * E >= (1ll << 31) || static_cast<long long>(T) * H >= (1ll << 40))
        return MOE_ERR_BAD_SHAPE;
    if (!std::isfinite(scale)) return MOE_ERR_BAD_ARG;
    if (T == 0) return MOE_OK;
    if (!bias || !token_mask || !logits || !topk_ids || !topk_w) return MOE_ERR_NULL_ARG;
    if (!logits_in && !W) return MOE_ERR_NULL_ARG;
    if (!all_aligned16(hidden, W, bias, token_mask, logits, topk_ids, topk_w)) return MOE_ERR_ALIGN;
    if (logits_in)
        return run_select(nullptr, 0, 1.f, 1, bias, token_mask, T, E, k, logits, topk_ids, topk_w, stream);

    const size_t need = moe_route_workspace_bytes(T, H, E, k, hidden_dtype, 0);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    const RoutePlan p = plan_route(T, H, E, hidden_dtype);
    char* ws = static_cast<char*>(workspace);
    uint16_t* w_planes = reinterpret_cast<uint16_t*>(ws);
    uint16_t* a_planes = reinterpret_cast<uint16_t*>(ws + p.w_planes_bytes);
    float* partials = reinterpret_cast<float*>(ws + p.w_planes_bytes + p.a_planes_bytes);

    const int cus = device_cu_count();
    const size_t wn = static_cast<size_t>(E) * H;
    int rc = launch(split3_kernel, dim3(ceil_div(static_cast<long long>(wn), 256 * 4) < cus * 8 ? ceil_div(static_cast<long long>(wn), 256 * 4) : cus * 8),
                    dim3(256), 0, stream, W, wn, w_planes);
    if (rc) return rc;
    const dim3 grid(p.tiles_n, p.tiles_m, p.nsplit);
    if (hidden_dtype == MOE_DTYPE_F32) {
        const size_t an = static_cast<size_t>(T) * H;
        rc = launch(split3_kernel, dim3(ceil_div(static_cast<long long>(an), 256 * 4) < cus * 8 ? ceil_div(static_cast<long long>(an), 256 * 4) : cus * 8),
                    dim3(256), 0, stream, static_cast<const float*>(hidden), an, a_planes);
        if (rc) return rc;
        rc = launch(proj_kernel<3>, grid, dim3(kGemmBlock), 0, stream,
                    static_cast<const uint16_t*>(a_planes), static_cast<const uint16_t*>(w_planes),
                    T, H, E, p.kslice, partials);
    } else {
        rc = launch(proj_kernel<1>, grid, dim3(kGemmBlock), 0, stream,
                    static_cast<const uint16_t*>(hidden), static_cast<const uint16_t*>(w_planes),
                    T, H, E, p.kslice, partials);
    }
    if (rc) return rc;
    return run_select(partials, p.nsplit, scale, 0, bias, token_mask, T, E, k, logits, topk_ids,
                      topk_w, stream);
}
