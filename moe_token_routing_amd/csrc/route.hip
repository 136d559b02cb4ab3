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
//    holds the next 8 significant bits of what the previous ones missed, to
//    nearest even; for |W| >= 2^-100 the sum is exact). A BF16 input times a
//    BF16 plane is exact in FP32, so the three MFMA products h*W0 + h*W1 +
//    h*W2 accumulate exact products of the FP32 weights in FP32
//    (v_mfma_f32_32x32x16_bf16). An FP32 input is split the same way (by a
//    kernel of its own, into planes in HBM) and the six products with
//    plane-index sum <= 2 are accumulated (the three dropped ones are below
//    2^-23 of |h*W|).
//  * Where the weights are split depends on the kernel: each wave loads the
//    FP32 weights themselves, 8 consecutive K values of one expert per lane
//    (the B operand's layout), and splits them in registers
//    (v_cvt_pk_bf16_f32, two values at a time) -- in the pipelined kernel
//    for large batches, where the split hides under the MFMAs and the FP32
//    weights are 2/3 of the bytes of three planes, and in the 128-token-tile
//    kernel below 4096 tokens; that kernel from 4096 tokens instead reads
//    planes a kernel of their own writes once per call in MFMA fragment
//    order (one 16-byte load per fragment). Both give the same planes.
//  * Block tile up to 128 tokens x 256 experts (all of them at E = 256, so the
//    input is read from HBM once), four waves of up to 128 x 64. The input
//    rows, shared by the four waves, go through a ring of LDS stages filled
//    by direct-to-LDS loads; the weights go straight to registers, one K-step
//    ahead. Split-K when the tile grid alone cannot fill the GPU, arranged so
//    that each XCD reads one K-slice of the weights (which then stays in its
//    L2). Partial sums go to the workspace.
//  * The selection (select.hip) adds the split-K partials in a fixed order,
//    applies the scale and picks the top k.
#include <cmath>

#include "dispatch.hpp"
#include "launch.hpp"
#include "select.hpp"

namespace moe {
namespace {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));

constexpr int kTargetBlocks = 480;        // about two blocks per CU
constexpr int kTargetBlocksSmall = 256;   // one block per CU (batches of up to 256 tokens)
constexpr int kPipeTargetBlocks = 256;   // one block per CU (proj_pipe_kernel)
#ifndef MOE_PIPE_SPLIT_IN_REGS
#define MOE_PIPE_SPLIT_IN_REGS 1
#endif
constexpr bool kPipeSplitInRegs = MOE_PIPE_SPLIT_IN_REGS;

// Zeroes p[0, n) over the whole grid: the per-tile expert histograms that
// the fused route + dispatch's selection counts into (run by the projection,
// which precedes the selection on the stream, after its own stores).
__device__ __forceinline__ void clear_range(int32_t* __restrict__ p, long long n) {
    for (long long i = blockIdx.x * static_cast<long long>(blockDim.x) + threadIdx.x; i < n;
         i += static_cast<long long>(gridDim.x) * blockDim.x)
        p[i] = 0;
}

// ---------------------------------------------------------------- split ----

// x (FP32) -> three BF16 values whose sum is x (each the next 8 significant
// bits of what the previous ones missed).
__device__ __forceinline__ void split3(float v, uint32_t& p0, uint32_t& p1, uint32_t& p2) {
    p0 = f32_to_bf16_rne(v);
    const float r1 = v - __uint_as_float(p0 << 16);
    p1 = f32_to_bf16_rne(r1);
    const float r2 = r1 - __uint_as_float(p1 << 16);
    p2 = f32_to_bf16_rne(r2);
}

// FP32 input rows -> three BF16 planes [3][n] in the input's own layout.
__global__ __launch_bounds__(256) void split3_kernel(const float* __restrict__ x, size_t n,
                                                     uint16_t* __restrict__ planes) {
    const size_t stride = static_cast<size_t>(gridDim.x) * blockDim.x;
    for (size_t i = static_cast<size_t>(blockIdx.x) * blockDim.x + threadIdx.x; i < n; i += stride) {
        uint32_t p0, p1, p2;
        split3(x[i], p0, p1, p2);
        planes[i] = static_cast<uint16_t>(p0);
        planes[n + i] = static_cast<uint16_t>(p1);
        planes[2 * n + i] = static_cast<uint16_t>(p2);
    }
}

__device__ __forceinline__ int swz(int row) { return ((row >> 2) ^ (row >> 3)) & 1; }
__device__ __forceinline__ int slot_bytes(int row, int c) { return (row * 2 + (c ^ swz(row))) * 16; }

// Router weight [E,H] FP32 -> its three BF16 planes as MFMA B fragments.
// For expert tile j (BN = 32 G experts) and K-step s (16 columns), one
// contiguous run of 3 G fragments of 1 KB, fragment (plane p, group g) at
// index p G + g; lane l of a fragment holds 8 consecutive K values
// [16 s + 8 (l >> 5), +8) of expert 32 (G j + g) + (l & 31) -- exactly the
// B operand of v_mfma_f32_32x32x16_bf16 for those 32 experts, so one wave
// loads a fragment with one 16-byte load per lane. Experts beyond E are zero.
//
// One thread per fragment lane and K-step: it reads its 8 FP32 weights once
// (32 bytes) and writes their three planes, so each wave writes three 1 KB
// runs.
__global__ __launch_bounds__(256) void split_weight_kernel(const float* __restrict__ W, int E, int H,
                                                           int G, int tiles_n,
                                                           u32x4* __restrict__ frags) {
    const int nks = H / 16;
    const int per_step = G * 64;                       // (group, lane) pairs of one plane
    const long long total = static_cast<long long>(tiles_n) * nks * per_step;
    const long long stride = static_cast<long long>(gridDim.x) * blockDim.x;
    for (long long s = static_cast<long long>(blockIdx.x) * blockDim.x + threadIdx.x; s < total; s += stride) {
        const long long blk = s / per_step;            // tile * nks + K-step
        const int sl = static_cast<int>(s - blk * per_step);
        const int tile = static_cast<int>(blk / nks);
        const int ks = static_cast<int>(blk - static_cast<long long>(tile) * nks);
        const int g = sl >> 6, l = sl & 63;
        const int e = (tile * G + g) * 32 + (l & 31);
        uint32_t h[3][8];
#pragma unroll
        for (int p = 0; p < 3; ++p)
#pragma unroll
            for (int j = 0; j < 8; ++j) h[p][j] = 0u;
        if (e < E) {
            const float4* src = reinterpret_cast<const float4*>(W + static_cast<size_t>(e) * H + ks * 16 + (l >> 5) * 8);
            const float4 a = src[0], b = src[1];
            const float v[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
            for (int j = 0; j < 8; ++j) split3(v[j], h[0][j], h[1][j], h[2][j]);
        }
        u32x4* out = frags + blk * (3 * per_step) + sl;
#pragma unroll
        for (int p = 0; p < 3; ++p)
            out[p * per_step] = u32x4{h[p][0] | (h[p][1] << 16), h[p][2] | (h[p][3] << 16),
                                      h[p][4] | (h[p][5] << 16), h[p][6] | (h[p][7] << 16)};
    }
}

// ----------------------------------------------------------------- gemm ----

// Block tile: BM = 32*MT tokens x BN = 128*NT experts; four waves side by
// side along the experts, each computing 32*MT x 32*NT with MT x NT
// accumulators of v_mfma_f32_32x32x16_bf16. K advances in steps of 16 (one
// MFMA K-step).
//
// The waves of a block share the input rows but not the weights, so only the
// input goes through LDS: a ring of DA stages filled DA-1 steps ahead by
// direct-to-LDS 16-byte loads (global_load_lds_dwordx4: lane l writes bytes
// [16 l, 16 l + 16) of the instruction's 1 KB LDS window). Each wave loads its
// own weights (fragments, or FP32 values it splits at the step) straight
// into registers one step ahead (two register sets), which keeps the weight
// traffic out of LDS. Two blocks share a CU, so one block's
// waits overlap the other's MFMAs.
//
// LDS stage layout: rows of 16 BF16 (two 16-byte chunks), NA planes x BM
// rows. Chunk c of row R sits in slot 2 R + (c ^ swz(R)),
// swz(R) = ((R >> 2) ^ (R >> 3)) & 1, so the 16 (or 8) lanes that read one
// chunk of 16 (or 8) consecutive rows in one LDS cycle touch distinct banks.
constexpr int kKC = 16;
constexpr int kGemmBlock = 256;
constexpr int kGemmWaves = kGemmBlock / kWave;
constexpr int kARing = 8;   // input stages in flight

template <int NA, int MT, int NT>
struct GemmShape {
    static constexpr int BM = 32 * MT;
    static constexpr int BN = 128 * NT;
    static constexpr int A_ROWS = NA * BM;
    static constexpr int A_LOADS = A_ROWS * 2 / kWave;   // 1 KB load instructions per stage
    static constexpr int STAGE = A_ROWS * 32;            // bytes
    static constexpr size_t LDS = static_cast<size_t>(kARing) * STAGE;
};

// Input rows [m0, m0 + BM) x K columns [k0, k0 + 16) of every input plane into
// the stage buffer at `base`; rows beyond T read row T - 1 (their results
// are never stored).
template <typename S>
__device__ __forceinline__ void issue_a(char* base, int k0, int wave, int lane, int m0, int T, int H,
                                        const uint16_t* __restrict__ a_planes, size_t a_plane) {
    const int lr = lane >> 1;
    const int sc = lane & 1;
    for (int i = wave; i < S::A_LOADS; i += kGemmWaves) {
        const int R = i * 32 + lr;
        const int c = sc ^ swz(R);
        const int p = R / S::BM, r = R - p * S::BM;
        const int row = min(m0 + r, T - 1);
        const uint16_t* src = a_planes + p * a_plane + static_cast<size_t>(row) * H + k0 + c * 8;
        __builtin_amdgcn_global_load_lds(src, base + i * 1024, 16, 0, 0);
    }
}

// Eight FP32 weights (two float4) -> their three BF16 planes as MFMA B
// fragments: W = W0 + W1 + W2 exactly, each plane the round-to-nearest-even
// BF16 of what the previous planes left.
__device__ __forceinline__ void split_fragment(const float4 (&w)[2], bf16x8_t& b0, bf16x8_t& b1, bf16x8_t& b2) {
    const float v[8] = {w[0].x, w[0].y, w[0].z, w[0].w, w[1].x, w[1].y, w[1].z, w[1].w};
    u32x4 q0, q1, q2;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const float x0 = v[2 * j], x1 = v[2 * j + 1];
        const uint32_t p0 = cvt_pk_bf16(x0, x1);
        const float r0 = x0 - bf16_lo(p0), r1 = x1 - bf16_hi(p0);
        const uint32_t p1 = cvt_pk_bf16(r0, r1);
        const uint32_t p2 = cvt_pk_bf16(r0 - bf16_lo(p1), r1 - bf16_hi(p1));
        q0[j] = p0;
        q1[j] = p1;
        q2[j] = p2;
    }
    b0 = __builtin_bit_cast(bf16x8_t, q0);
    b1 = __builtin_bit_cast(bf16x8_t, q1);
    b2 = __builtin_bit_cast(bf16x8_t, q2);
}

// Block b works on K-slice b % nsplit and tile b / nsplit. Blocks go to the
// eight XCDs round-robin, so when nsplit divides 8 every XCD only ever reads
// one K-slice of the weights and keeps it in its own L2.
//
// PRESPLIT: the weights come as split_weight_kernel's fragment-ordered
// planes (w_frags), one 16-byte load per lane and fragment. Otherwise they
// come as the FP32 rows of W and each wave splits its own: for many tokens
// the split, repeated by every row tile, costs the MFMA loop more (about 7%
// at 4096-8192 tokens) than one split kernel per call, for few tokens less.
template <int NA, int MT, int NT, bool PRESPLIT>
__global__ __launch_bounds__(kGemmBlock) __attribute__((amdgpu_waves_per_eu(2))) void proj_kernel(
    const uint16_t* __restrict__ a_planes, const float* __restrict__ W, const uint16_t* __restrict__ w_frags,
    int T, int H, int E, int kslice, int nsplit, int tiles_m, float* __restrict__ partials,
    int32_t* __restrict__ clear, long long clear_n) {
    using S = GemmShape<NA, MT, NT>;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x;
    const int lane = __lane_id();
    const int wave = tid / kWave;
    const int split = blockIdx.x % nsplit;
    const int tile = blockIdx.x / nsplit;
    const int m0 = (tile % tiles_m) * S::BM;
    const int n_tile = tile / tiles_m;
    const int n0 = n_tile * S::BN;
    const int kbeg = split * kslice;
    const int kend = min(H, kbeg + kslice);
    const int nst = (kend - kbeg) / kKC;
    const size_t a_plane = static_cast<size_t>(T) * H;

    f32x16_t acc[MT][NT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt)
#pragma unroll
            for (int i = 0; i < 16; ++i) acc[mt][nt][i] = 0.f;

    const int frow = lane & 31;
    const int c = lane >> 5;   // chunk: K columns [8c, 8c + 8) of the step
    // B operand of accumulator column group nt: expert n0 + 32 (wave NT + nt)
    // + (lane & 31), K columns [16 s + 8 c, +8) of step s; experts past E
    // read expert E - 1 (their results are never stored)
    const float* wrow[NT];
#pragma unroll
    for (int nt = 0; nt < NT; ++nt) {
        const int e = min(n0 + (wave * NT + nt) * 32 + frow, E - 1);
        wrow[nt] = W + static_cast<size_t>(e) * H + kbeg + 8 * c;
    }
    float4 wq[2][NT][2];      // FP32 weights of two steps
    bf16x8_t bq[2][3][NT];    // (PRESPLIT) fragments of two steps
    // this tile's fragments, from the first K-step of the slice
    constexpr int G = S::BN / 32;   // fragments per plane and K-step
    const bf16x8_t* frags = reinterpret_cast<const bf16x8_t*>(w_frags) +
                            (static_cast<size_t>(n_tile) * (H / kKC) + kbeg / kKC) * (3 * G * kWave);
    auto load_b = [&](int s, int set) {
        if constexpr (PRESPLIT) {
            const bf16x8_t* src = frags + static_cast<size_t>(s) * (3 * G * kWave);
#pragma unroll
            for (int p = 0; p < 3; ++p)
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) bq[set][p][nt] = src[(p * G + wave * NT + nt) * kWave + lane];
        } else {
#pragma unroll
            for (int nt = 0; nt < NT; ++nt) {
                const float4* src = reinterpret_cast<const float4*>(wrow[nt] + s * kKC);
                wq[set][nt][0] = src[0];
                wq[set][nt][1] = src[1];
            }
        }
    };

    if (nst > 0) load_b(0, 0);
    for (int s = 0; s < kARing - 1 && s < nst; ++s)
        issue_a<S>(lds + s * S::STAGE, kbeg + s * kKC, wave, lane, m0, T, H, a_planes, a_plane);
    for (int s0 = 0; s0 < nst; s0 += 2) {
#pragma unroll
        for (int ph = 0; ph < 2; ++ph) {
            const int s = s0 + ph;
            if (s < nst) {
                // every load of this wave has landed (stage s included), then
                // every wave's: stage s is complete and stage s-1 is free
                __builtin_amdgcn_s_waitcnt(0);
                __syncthreads();
                bf16x8_t b[3][NT];
#pragma unroll
                for (int nt = 0; nt < NT; ++nt) {
                    if constexpr (PRESPLIT) {
#pragma unroll
                        for (int p = 0; p < 3; ++p) b[p][nt] = bq[ph][p][nt];
                    } else {
                        split_fragment(wq[ph][nt], b[0][nt], b[1][nt], b[2][nt]);
                    }
                }
                if (s + 1 < nst) load_b(s + 1, ph ^ 1);
                if (s + kARing - 1 < nst)
                    issue_a<S>(lds + ((s + kARing - 1) % kARing) * S::STAGE, kbeg + (s + kARing - 1) * kKC,
                               wave, lane, m0, T, H, a_planes, a_plane);
                const char* base = lds + (s % kARing) * S::STAGE;
                bf16x8_t a[NA][MT];
#pragma unroll
                for (int p = 0; p < NA; ++p)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
                        a[p][mt] = *reinterpret_cast<const bf16x8_t*>(base + slot_bytes(p * S::BM + mt * 32 + frow, c));
                // products (input plane, weight plane) in the outer loop, so
                // that consecutive MFMAs write different accumulators
                constexpr int NPROD = NA == 1 ? 3 : 6;
                constexpr int PA[6] = {0, 0, 0, 1, 1, 2};
                constexpr int PB[6] = {0, 1, 2, 0, 1, 0};
#pragma unroll
                for (int q = 0; q < NPROD; ++q)
#pragma unroll
                    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                        for (int nt = 0; nt < NT; ++nt)
                            acc[mt][nt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a[PA[q]][mt], b[PB[q]][nt],
                                                                                  acc[mt][nt], 0, 0, 0);
            }
        }
    }

    // 32x32 accumulator layout: lane holds column (lane & 31) and rows
    // 8*(i/4) + 4*(lane/32) + (i%4) for i = 0..15.
    float* out = partials + static_cast<size_t>(split) * T * E;
    const int half = lane >> 5;
#pragma unroll
    for (int mt = 0; mt < MT; ++mt)
#pragma unroll
        for (int nt = 0; nt < NT; ++nt) {
            const int col = n0 + (wave * NT + nt) * 32 + (lane & 31);
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + mt * 32 + 8 * (i >> 2) + 4 * half + (i & 3);
                if (row < T && col < E) out[static_cast<size_t>(row) * E + col] = acc[mt][nt][i];
            }
        }
    clear_range(clear, clear_n);
}

// ------------------------------------------------------ pipelined gemm ----

// The projection for large batches (BF16 input, weights split by
// split_weight_kernel), software-pipelined so that no step waits for a load
// issued in the previous one.
//
// Block tile: 256 tokens x 256 experts, eight waves side by side along the
// experts, each 256 x 32 (eight v_mfma_f32_32x32x16_bf16 accumulators); one
// block per CU (two waves per SIMD). Per block, a 256-token tile reads each
// weight fragment once for twice as many tokens as a 128-token tile, which
// halves the L2 -> CU weight traffic.
//
// Pipeline: every K-step s issues one group of loads for step s + kLook -- one
// direct-to-LDS 16-byte load of the input stage per wave (the eight waves
// fill the 8 KB stage of 256 rows x 16 columns) and the wave's weights into
// one of kLook + 1 register sets: two 16-byte loads of FP32 weights, split
// into the three BF16 planes at the step that uses them (FP32W; measured
// 101 -> 98 us at 8192 tokens and no split kernel), or three 16-byte
// fragments of the split kernel's planes.
// Loads complete in issue order, so waiting until at most (kLook - 1) groups
// are outstanding (s_waitcnt vmcnt) means step s's group has landed while
// the next kLook - 1 stay in flight; a barrier without a memory fence then
// makes every wave's part of the input stage visible. The LDS ring has
// kLook + 1 stages: the stage refilled at step s is the one all waves finished
// reading before that barrier. The loop is unrolled over the register sets
// and nothing is issued conditionally inside it (loads past the last step
// repeat the last step's addresses into a set and a stage nobody reads), so
// the compiler's own wait placement stays exact.
constexpr int kPipeWaves = 8;
constexpr int kPipeBlock = kPipeWaves * kWave;
constexpr int kPipeMT = 8;                       // 32-token row groups per wave
constexpr int kPipeBM = 32 * kPipeMT;            // 256 tokens
constexpr int kPipeBN = 32 * kPipeWaves;         // 256 experts
constexpr int kLook = 3;                         // steps of loads in flight
constexpr int kPipeSets = kLook + 1;             // register sets = LDS stages
constexpr int kPipeStage = kPipeBM * 32;         // 8 KB: 256 rows x 16 BF16
constexpr size_t kPipeLds = static_cast<size_t>(kPipeSets) * kPipeStage;
static_assert(kPipeBM * 2 / kWave == kPipeWaves, "one input load per wave and step");
static_assert(kPipeSets == 4, "the main loop is unrolled over four sets");

// s_waitcnt with only the vector-memory count constrained (expcnt and
// lgkmcnt at their maxima), for gfx9's split vmcnt field.
template <int N>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xF) | ((N >> 4) << 14) | (0x7 << 4) | (0xF << 8));
}

// Block b works on K-slice b % nsplit (each XCD keeps one slice of the
// weight planes in its L2 when nsplit divides 8) and token tile b / nsplit;
// the expert tile is tile / tiles_m. Requires (kend - kbeg) to be a positive
// multiple of 64 for every slice (plan_route checks it).
template <bool FP32W>
__global__ __launch_bounds__(kPipeBlock) __attribute__((amdgpu_waves_per_eu(2))) void proj_pipe_kernel(
    const uint16_t* __restrict__ a, const float* __restrict__ W, const uint16_t* __restrict__ w_frags, int T,
    int H, int E, int kslice, int nsplit, int tiles_m, float* __restrict__ partials,
    int32_t* __restrict__ clear, long long clear_n) {
    constexpr int kLoads = FP32W ? 3 : 4;   // loads per wave and step: the input, then the weights
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int split = blockIdx.x % nsplit;
    const int tile = blockIdx.x / nsplit;
    const int m0 = (tile % tiles_m) * kPipeBM;
    const int n_tile = tile / tiles_m;
    const int kbeg = split * kslice;
    const int nst = (min(H, kbeg + kslice) - kbeg) / kKC;

    f32x16_t acc[kPipeMT];
#pragma unroll
    for (int mt = 0; mt < kPipeMT; ++mt)
#pragma unroll
        for (int i = 0; i < 16; ++i) acc[mt][i] = 0.f;

    // this wave's input load: rows 32 wave + lane / 2 of the tile, chunk
    // (lane & 1) ^ swz(row) of the stage's 16 columns (rows past T read row
    // T - 1, whose results are never stored)
    const int a_row = wave * 32 + (lane >> 1);
    const int a_chunk = (lane & 1) ^ swz(a_row);
    const uint16_t* a_src = a + static_cast<size_t>(min(m0 + a_row, T - 1)) * H + kbeg + a_chunk * 8;
    char* a_dst = lds + wave * 1024;
    // this wave's weight fragments: group `wave` of the tile's run for each
    // K-step (3 planes x 8 groups x 64 lanes of 16 bytes)
    constexpr int G = kPipeBN / 32;
    const bf16x8_t* b_src = reinterpret_cast<const bf16x8_t*>(w_frags) +
                            (static_cast<size_t>(n_tile) * (H / kKC) + kbeg / kKC) * (3 * G * kWave) +
                            wave * kWave + lane;
    bf16x8_t bq[kPipeSets][3];
    // FP32W: the wave's FP32 weights themselves, 8 consecutive K values of
    // expert (lane & 31) per lane (the B operand's layout; experts past E read
    // expert E - 1, whose results are never stored), split into the three
    // BF16 planes in registers when used
    const float* w_src = W + static_cast<size_t>(min(n_tile * kPipeBN + wave * 32 + (lane & 31), E - 1)) * H +
                         kbeg + 8 * (lane >> 5);
    float4 wq[kPipeSets][2];
    // The blocks of one XCD run the same K-slice in step: each starts its walk
    // over the slice at an offset of its own (two K-steps per token tile) so
    // that at any moment they read different lines of the shared weight
    // planes instead of the same few (-7% at 8192 tokens). The order of a
    // block's additions is fixed, so results stay reproducible.
    const int rot = ((tile % tiles_m) * 2) % max(nst, 1);

    auto issue = [&](int step, int set) {
        const int s = step + rot < nst ? step + rot : step + rot - nst;
        __builtin_amdgcn_global_load_lds(a_src + s * kKC, a_dst + set * kPipeStage, 16, 0, 0);
        if constexpr (FP32W) {
            const float4* src = reinterpret_cast<const float4*>(w_src + s * kKC);
            wq[set][0] = src[0];
            wq[set][1] = src[1];
        } else {
#pragma unroll
            for (int p = 0; p < 3; ++p) bq[set][p] = b_src[static_cast<size_t>(s) * (3 * G * kWave) + p * G * kWave];
        }
    };

    if (nst > 0) {
#pragma unroll
        for (int s = 0; s < kLook; ++s) {
            issue(s, s);
            __builtin_amdgcn_sched_barrier(0);
        }
        int s0 = 0;
        do {
#pragma unroll
            for (int ph = 0; ph < kPipeSets; ++ph) {
                const int s = s0 + ph;
                __builtin_amdgcn_sched_barrier(0);
                wait_vmcnt<(kLook - 1) * kLoads>();   // step s's loads have landed
                __builtin_amdgcn_s_barrier();              // ... in every wave
                __builtin_amdgcn_sched_barrier(0);
                issue(min(s + kLook, nst - 1), (ph + kLook) % kPipeSets);
                __builtin_amdgcn_sched_barrier(0);
                const char* base = lds + ph * kPipeStage;
                bf16x8_t av[kPipeMT];
#pragma unroll
                for (int mt = 0; mt < kPipeMT; ++mt)
                    av[mt] = *reinterpret_cast<const bf16x8_t*>(base + slot_bytes(mt * 32 + (lane & 31), lane >> 5));
                bf16x8_t b[3];
                if constexpr (FP32W) {
                    split_fragment(wq[ph], b[0], b[1], b[2]);
                } else {
#pragma unroll
                    for (int p = 0; p < 3; ++p) b[p] = bq[ph][p];
                }
#pragma unroll
                for (int p = 0; p < 3; ++p)
#pragma unroll
                    for (int mt = 0; mt < kPipeMT; ++mt)
                        acc[mt] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(av[mt], b[p], acc[mt], 0, 0, 0);
            }
            s0 += kPipeSets;
        } while (s0 < nst);
        wait_vmcnt<0>();   // the repeated loads of the last steps, before the wave ends
    }

    // accumulator layout: lane holds expert column (lane & 31) and token rows
    // 8 (i / 4) + 4 (lane / 32) + (i % 4), i = 0..15
    float* out = partials + static_cast<size_t>(split) * T * E;
    const int col = n_tile * kPipeBN + wave * 32 + (lane & 31);
    if (col < E) {
#pragma unroll
        for (int mt = 0; mt < kPipeMT; ++mt)
#pragma unroll
            for (int i = 0; i < 16; ++i) {
                const int row = m0 + mt * 32 + 8 * (i >> 2) + 4 * (lane >> 5) + (i & 3);
                if (row < T) out[static_cast<size_t>(row) * E + col] = acc[mt][i];
            }
    }
    clear_range(clear, clear_n);
}

// From this many tokens the weights are split once per call into
// fragment-ordered planes; below, each wave splits the FP32 weights it loads.
constexpr int kPresplitTokens = 4096;

// Workspace layout: [W planes (from kPresplitTokens)][input planes (FP32
// input)][partials].
struct RoutePlan {
    int na, mt, nt;                 // kernel variant
    bool presplit;
    bool pipe;                      // proj_pipe_kernel (256 x 256 tiles) instead of proj_kernel
    int tiles_m, tiles_n, nsplit, kslice;
    size_t w_planes_bytes, a_planes_bytes, partial_bytes;
};

inline size_t round256(size_t b) { return (b + 255) / 256 * 256; }

// Tile shape and split-K count are functions of (T, H, E, dtype) only, so
// the workspace query and the call always agree.
inline RoutePlan plan_route(int T, int H, int E, int hidden_dtype) {
    RoutePlan p;
    p.na = hidden_dtype == MOE_DTYPE_F32 ? 3 : 1;
    // 256-expert tiles, except for small batches (up to 256 tokens), whose
    // blocks are latency-bound with one wave a SIMD: 128-expert tiles double
    // the blocks and halve each wave's weight split (at 128 tokens of 8192 x
    // 256 the step replayed from a graph 39.7 -> 38.9 us)
    p.nt = E > 128 && T > 256 ? 2 : 1;
    p.mt = T >= 2048 ? 4 : (T >= 256 ? 2 : 1);
    if (p.na == 3 && p.mt > 2) p.mt = 2;   // three input planes: keep the registers of two blocks per CU
    p.tiles_m = ceil_div(T, 32 * p.mt);
    p.tiles_n = ceil_div(E, 128 * p.nt);
    const int tiles = p.tiles_m * p.tiles_n;
    const int chunks = ceil_div(H, kKC);
    // split K until about two blocks a CU; small batches stop at one a CU,
    // whose blocks then run twice the K-steps against half the partials
    // (at 128 tokens of 8192 x 256: split 64 -> 32, projection 10.6 -> 10.1
    // us, selection 6.2 -> 5.2 us; split 16 took 14 us)
    const int target = T <= 256 ? kTargetBlocksSmall : kTargetBlocks;
    int ns = 1;
    while (tiles * ns < target && ns * 2 <= chunks && ns < 64) ns *= 2;
    const int per = ceil_div(chunks, ns);   // K stages per split
    p.kslice = per * kKC;
    p.nsplit = ceil_div(H, p.kslice);
    p.presplit = T >= kPresplitTokens;
    p.pipe = false;
    // large batches of BF16 input whose K-steps divide into whole unrolled
    // rounds of four: the pipelined kernel
    // (one block per CU), when its grid is a whole number of GPU-fulls;
    // otherwise (a last partial wave of blocks) the two-blocks-per-CU kernel
    // balances better
    if (p.presplit && p.na == 1 && H % (4 * kKC) == 0) {
        const int tm = ceil_div(T, kPipeBM), tn = ceil_div(E, kPipeBN);
        const int rounds = H / (4 * kKC);           // unrolled rounds of four K-steps
        int n = 1;
        while (tm * tn * n < kPipeTargetBlocks && n * 2 <= rounds && n < 64) n *= 2;
        const int kslice = ceil_div(rounds, n) * 4 * kKC;
        const int nsplit = ceil_div(H, kslice);
        if ((tm * tn * nsplit) % kPipeTargetBlocks == 0) {
            p.pipe = true;
            p.presplit = !kPipeSplitInRegs;
            p.nt = 2;                               // fragment groups of 256-expert tiles
            p.tiles_m = tm;
            p.tiles_n = tn;
            p.kslice = kslice;
            p.nsplit = nsplit;
        }
    }
    // fragment-ordered planes, padded to whole expert tiles
    p.w_planes_bytes = p.presplit ? round256(static_cast<size_t>(3) * p.tiles_n * 128 * p.nt * H * sizeof(uint16_t)) : 0;
    p.a_planes_bytes = p.na == 3 ? round256(static_cast<size_t>(3) * T * H * sizeof(uint16_t)) : 0;
    p.partial_bytes = round256(static_cast<size_t>(p.nsplit) * T * E * sizeof(float));
    return p;
}

template <int NA, int MT, int NT>
int launch_proj(const RoutePlan& p, const uint16_t* a, const float* W, const uint16_t* w_frags, int T, int H,
                int E, float* partials, int32_t* clear, long long clear_n, void* stream) {
    using S = GemmShape<NA, MT, NT>;
    const dim3 grid(p.tiles_m * p.tiles_n * p.nsplit);
    if (p.presplit)
        return launch(proj_kernel<NA, MT, NT, true>, grid, dim3(kGemmBlock), S::LDS, stream, a, W, w_frags, T, H,
                      E, p.kslice, p.nsplit, p.tiles_m, partials, clear, clear_n);
    return launch(proj_kernel<NA, MT, NT, false>, grid, dim3(kGemmBlock), S::LDS, stream, a, W, w_frags, T, H, E,
                  p.kslice, p.nsplit, p.tiles_m, partials, clear, clear_n);
}

// The projection's launch; it also zeroes clear[0, clear_n) (nothing when
// clear_n is 0).
int run_proj(const RoutePlan& p, const uint16_t* a, const float* W, const uint16_t* w_frags, int T, int H,
             int E, float* partials, int32_t* clear, long long clear_n, void* stream) {
    if (p.pipe) {
        const dim3 grid(p.tiles_m * p.tiles_n * p.nsplit);
        if (!p.presplit)
            return launch(proj_pipe_kernel<true>, grid, dim3(kPipeBlock), kPipeLds, stream, a, W, w_frags, T, H, E,
                          p.kslice, p.nsplit, p.tiles_m, partials, clear, clear_n);
        return launch(proj_pipe_kernel<false>, grid, dim3(kPipeBlock), kPipeLds, stream, a, W, w_frags, T, H, E,
                      p.kslice, p.nsplit, p.tiles_m, partials, clear, clear_n);
    }
#define MOE_PROJ(NA, MT, NT) \
    if (p.na == NA && p.mt == MT && p.nt == NT) \
        return launch_proj<NA, MT, NT>(p, a, W, w_frags, T, H, E, partials, clear, clear_n, stream);
    MOE_PROJ(1, 1, 1) MOE_PROJ(1, 1, 2) MOE_PROJ(1, 2, 1) MOE_PROJ(1, 2, 2) MOE_PROJ(1, 4, 1) MOE_PROJ(1, 4, 2)
    MOE_PROJ(3, 1, 1) MOE_PROJ(3, 1, 2) MOE_PROJ(3, 2, 1) MOE_PROJ(3, 2, 2)
#undef MOE_PROJ
    return MOE_ERR_BAD_SHAPE;
}

// Argument checks of moe_route (before any launch); a moe_status.
int check_route(const void* hidden, int hidden_dtype, const float* W, const float* bias, const uint8_t* token_mask,
                float scale, int T, int H, int E, int k, const float* logits, const int32_t* topk_ids,
                const float* topk_w) {
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
    return MOE_OK;
}

// The route's launches for T > 0 on checked arguments and a large enough
// workspace. With hist set (hist_n int32 of per-tile expert histograms of
// hist_tile slots each), the histograms are zeroed and the selection counts
// every valid pick into them.
int run_route(const void* hidden, int hidden_dtype, const float* W, const float* bias, const uint8_t* token_mask,
              float scale, int T, int H, int E, int k, float* logits, int32_t* topk_ids, float* topk_w,
              void* workspace, int32_t* hist, long long hist_n, int hist_tile, void* stream) {
    if (hidden == nullptr) {   // logits in: the selection only
        if (hist) {
            const int rc = run_clear(hist, hist_n, stream);
            if (rc) return rc;
        }
        return run_select(nullptr, 0, 1.f, 1, bias, token_mask, T, E, k, logits, topk_ids, topk_w, hist,
                          hist_tile, stream);
    }
    const RoutePlan p = plan_route(T, H, E, hidden_dtype);
    char* ws = static_cast<char*>(workspace);
    uint16_t* w_planes = reinterpret_cast<uint16_t*>(ws);
    uint16_t* a_planes = reinterpret_cast<uint16_t*>(ws + p.w_planes_bytes);
    float* partials = reinterpret_cast<float*>(ws + p.w_planes_bytes + p.a_planes_bytes);

    const int cap = device_cu_count() * 8;
    if (p.presplit) {
        const int G = 4 * p.nt;   // 32-expert groups per expert tile
        const long long wslots = static_cast<long long>(p.tiles_n) * (H / kKC) * G * kWave;   // threads
        const int gw = ceil_div(wslots, 256);
        const int rc = launch(split_weight_kernel, dim3(gw < cap ? gw : cap), dim3(256), 0, stream, W, E, H, G,
                              p.tiles_n, reinterpret_cast<u32x4*>(w_planes));
        if (rc) return rc;
    }
    const uint16_t* a = static_cast<const uint16_t*>(hidden);
    if (p.na == 3) {
        const size_t an = static_cast<size_t>(T) * H;
        const int ga = ceil_div(static_cast<long long>(an), 256 * 4);
        const int rc = launch(split3_kernel, dim3(ga < cap ? ga : cap), dim3(256), 0, stream,
                              static_cast<const float*>(hidden), an, a_planes);
        if (rc) return rc;
        a = a_planes;
    }
    const int rc = run_proj(p, a, W, w_planes, T, H, E, partials, hist, hist ? hist_n : 0, stream);
    if (rc) return rc;
    return run_select(partials, p.nsplit, scale, 0, bias, token_mask, T, E, k, logits, topk_ids, topk_w, hist,
                      hist_tile, stream);
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
    const int rc = check_route(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids,
                               topk_w);
    if (rc || T == 0) return rc;
    if (hidden) {
        const size_t need = moe_route_workspace_bytes(T, H, E, k, hidden_dtype, 0);
        if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
        if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    }
    return run_route(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w,
                     workspace, nullptr, 0, 1, stream);
}

namespace {

// Bytes of the fused call's per-tile histograms (none with one tile).
size_t fused_hist_bytes(int T, int k, int E) {
    const long long n = static_cast<long long>(T) * k;
    if (n <= 0) return 0;
    const moe::DispatchTiles d = moe::dispatch_tiles(n);
    if (d.tiles <= 1) return 0;
    return (static_cast<size_t>(d.tiles) * E * sizeof(int32_t) + 255) / 256 * 256;
}

}  // namespace

extern "C" size_t moe_route_dispatch_workspace_bytes(int T, int H, int E, int k, int hidden_dtype,
                                                     int logits_in) {
    using namespace moe;
    if (T <= 0 || H <= 0 || E <= 0 || E > MOE_MAX_EXPERTS || k <= 0 || k > MOE_MAX_TOPK) return 0;
    if (!logits_in && hidden_dtype != MOE_DTYPE_F32 && hidden_dtype != MOE_DTYPE_BF16) return 0;
    return round256(moe_route_workspace_bytes(T, H, E, k, hidden_dtype, logits_in)) + fused_hist_bytes(T, k, E);
}

namespace moe {
namespace {

// The steps of moe_route_dispatch and moe_route_dispatch_quant (x == nullptr:
// no norm + quant; x is [T, Hq]) after their own argument checks.
int route_dispatch_run(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                       const uint8_t* token_mask, float scale, int T, int H, int E, int k, float* logits,
                       int32_t* topk_ids, float* topk_w, int32_t* counts, int32_t* offsets, int32_t* perm,
                       int32_t* dest, const uint16_t* x, int Hq, const float* norm_w, float gain_center, float eps,
                       const float* global_scale, uint8_t* packed, uint8_t* scales, void* workspace,
                       size_t workspace_bytes, void* stream) {
    if (T == 0) return run_dispatch_empty(counts, offsets, E, stream);
    const size_t route_bytes = round256(moe_route_workspace_bytes(T, H, E, k, hidden_dtype, hidden == nullptr));
    const size_t hist_bytes = fused_hist_bytes(T, k, E);
    if (route_bytes + hist_bytes > 0) {
        if (!workspace || workspace_bytes < route_bytes + hist_bytes) return MOE_ERR_WORKSPACE;
        if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    }
    const long long n = static_cast<long long>(T) * k;
    const DispatchTiles d = dispatch_tiles(n);
    int32_t* hist = hist_bytes ? reinterpret_cast<int32_t*>(static_cast<char*>(workspace) + route_bytes) : nullptr;
    const int rc = run_route(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w,
                             workspace, hist, static_cast<long long>(d.tiles) * E, d.tile, stream);
    if (rc) return rc;
    if (!x) return run_place(topk_ids, n, E, counts, offsets, perm, dest, hist, stream);
    return run_place_norm_quant(topk_ids, n, E, counts, offsets, perm, dest, hist, x, norm_w, gain_center, eps,
                                global_scale, T, Hq, packed, scales, stream);
}

}  // namespace
}  // namespace moe

extern "C" int moe_route_dispatch(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                                  const uint8_t* token_mask, float scale, int T, int H, int E, int k,
                                  float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                  int32_t* offsets, int32_t* perm, int32_t* dest, void* workspace,
                                  size_t workspace_bytes, void* stream) {
    using namespace moe;
    int rc = check_route(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w);
    if (rc) return rc;
    rc = check_dispatch(topk_ids, T, k, E, counts, offsets, perm, dest);
    if (rc) return rc;
    return route_dispatch_run(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w,
                              counts, offsets, perm, dest, nullptr, 0, nullptr, 0.f, 0.f, nullptr, nullptr, nullptr,
                              workspace, workspace_bytes, stream);
}

extern "C" int moe_route_dispatch_quant(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                                        const uint8_t* token_mask, float scale, int T, int H, int E, int k,
                                        float* logits, int32_t* topk_ids, float* topk_w, int32_t* counts,
                                        int32_t* offsets, int32_t* perm, int32_t* dest, const uint16_t* x,
                                        int Hq, const float* norm_w, float gain_center, float eps,
                                        const float* global_scale, uint8_t* packed, uint8_t* scales,
                                        void* workspace, size_t workspace_bytes, void* stream) {
    using namespace moe;
    int rc = check_route(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w);
    if (rc) return rc;
    rc = check_dispatch(topk_ids, T, k, E, counts, offsets, perm, dest);
    if (rc) return rc;
    rc = check_norm_quant(x, norm_w, gain_center, eps, global_scale, T, Hq, packed, scales);
    if (rc) return rc;
    return route_dispatch_run(hidden, hidden_dtype, W, bias, token_mask, scale, T, H, E, k, logits, topk_ids, topk_w,
                              counts, offsets, perm, dest, x, Hq, norm_w, gain_center, eps, global_scale, packed, scales,
                              workspace, workspace_bytes, stream);
}
