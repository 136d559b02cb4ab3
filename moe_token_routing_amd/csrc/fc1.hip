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
//    dequantised exactly to FP16: the unit-scale FP4 -> FP16 pair conversion
//    and one packed FP16 multiply by the E4M3 scale (a code value has at most
//    2 significant bits and a scale 4, so every product is exact and normal
//    in FP16). The GEMM then runs v_mfma_f32_32x32x16_f16 with FP32
//    accumulation (FP16 x FP16 products are exact in FP32); the global scales
//    are applied once, as alpha = 1 / (gs_x * gs_w[e]) in the epilogue.
//  * Block tile 256 grouped rows x 192 (or 256, or 128) output columns,
//    eight waves, so each dequantised row feeds more MFMAs.
//    K advances in stages of 64: the raw FP4 bytes of a stage are loaded
//    into registers two stages ahead (its scale bytes through LDS, below)
//    and dequantised, while the MFMAs of the stage before run, into the
//    other half of a double-buffered LDS tile (rows of 128 bytes, 16-byte
//    chunks XOR-swizzled so that neither access conflicts, chunk_off).
//  * The row tiles of each expert are laid out from `offsets` by a one-block
//    kernel (exclusive prefix of ceil(rows / 256) over experts, and one
//    16-byte record per tile: expert, first row, row end), so a GEMM block
//    learns its tile from one load; the grid is an upper bound, blocks past
//    the last tile leave at once. Blocks are remapped so that each XCD
//    walks a contiguous run of (row tile, column tile) with the column tile
//    fastest: the blocks of one gathered A tile run side by side and find it
//    in their XCD's L2, and so do an expert's weights across its row tiles.
//  * Epilogue straight from the accumulators: the MFMAs take the weight
//    rows as their first operand, so each lane holds 16 output columns of
//    one grouped row, half of two 16-column blocks; the two lanes holding a
//    block meet through v_permlane32_swap for its maximum and its codes.
//    alpha * acc, Relu2, then the pre-expert quantiser's FP32 steps
//    (hardware E4M3 and FP4 conversions, as there).
#include <cmath>

#include "launch.hpp"
#include "nvfp4.hpp"

namespace moe {
namespace {

typedef _Float16 f16x8_t __attribute__((ext_vector_type(8)));
typedef _Float16 f16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x16_t __attribute__((ext_vector_type(16)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kFcKS = 64;               // K per stage
constexpr int kFcTilesBlock = 512;      // threads of the tile-layout kernel
constexpr int kFcRaw = 2;               // stages of raw bytes in registers
constexpr int kFcSch = 8;               // stages per scale chunk: 4 scale bytes a stage, 32 a row

// Block tile BM x BN, WM x WN waves, each 32 MT x 32 NT; two threads per
// A row (each loads half of a stage's 64 K), and the B rows' halves spread
// over the threads NBI at a time.
template <int WM, int WN, int MT, int NT>
struct FcShape {
    static constexpr int BM = WM * MT * 32;
    static constexpr int BN = WN * NT * 32;
    static constexpr int THREADS = WM * WN * kWave;
    static_assert(THREADS == 2 * BM, "two threads per A row");
    static constexpr int NBI = (2 * BN + THREADS - 1) / THREADS;      // B row halves per thread
    static constexpr int STAGE = (BM + BN) * kFcKS * 2;              // A and B tiles, FP16 bytes
    static constexpr int SCHUNK = (BM + BN) * kFcSch * 4;             // one scale chunk of every row
    static constexpr size_t MAIN = 2 * static_cast<size_t>(STAGE) + 2 * static_cast<size_t>(SCHUNK);
    static constexpr size_t LDS = MAIN;
};

// Row tiles of `bm` rows over experts: at most ceil(P / bm) + E (each
// expert adds at most one partial tile).
inline long long fc1_row_tiles_upper(long long P, int E, int bm) { return (P + bm - 1) / bm + E; }

// tile_start[e] = sum over e' < e of ceil(rows(e') / bm); tile_start[E] =
// total. Row tile t of expert e (tile_start[e] <= t < tile_start[e + 1]) is
// described by tile_info[t] = (e, first grouped row, end of the expert's
// rows clamped to n_pos, 0), so a GEMM block finds its tile with one load.
__global__ __launch_bounds__(kFcTilesBlock) void fc1_tiles_kernel(const int32_t* __restrict__ offsets, int E,
                                                                  int n_pos, int bm, int m_upper,
                                                                  int32_t* __restrict__ tile_start,
                                                                  int4* __restrict__ tile_info) {
    __shared__ int32_t wsum[kFcTilesBlock / kWave];
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
    const int chunk = (E + kFcTilesBlock - 1) / kFcTilesBlock;
    const int e0 = min(E, tid * chunk), e1 = min(E, e0 + chunk);
    int local = 0;
    for (int e = e0; e < e1; ++e) local += (max(offsets[e + 1] - offsets[e], 0) + bm - 1) / bm;
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
        const int first = offsets[e], end = offsets[e + 1];
        const int n = (max(end - first, 0) + bm - 1) / bm;
        // (valid offsets never make more than m_upper tiles; others stop there)
        for (int i = 0; i < n && run + i < m_upper; ++i)
            tile_info[run + i] = make_int4(e, first + i * bm, min(end, n_pos), 0);
        run += n;
    }
    if (tid == kFcTilesBlock - 1) tile_start[E] = run;
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

// One 32-bit word (8 E2M1 codes) times its block scale -> 4 packed FP16
// pairs: the unit-scale FP4 -> FP16 conversion is exact, and so is the
// packed FP16 product (a code value has at most 2 significant bits, an E4M3
// scale 4, and every product lies in [2^-10, 2688], normal in FP16).
__device__ __forceinline__ uint32_t as_u32(f16x2_t v) {
    uint32_t u;
    __builtin_memcpy(&u, &v, 4);
    return u;
}
__device__ __forceinline__ void dequant8(uint32_t w, f16x2_t s2, uint32_t (&out)[4]) {
    out[0] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 0) * s2);
    out[1] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 1) * s2);
    out[2] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 2) * s2);
    out[3] = as_u32(__builtin_amdgcn_cvt_scalef32_pk_f16_fp4(w, 1.0f, 3) * s2);
}

// Block barrier that orders LDS accesses only: the wave waits for its own LDS
// operations (lgkmcnt 0), not for its global loads, which stay in flight
// across the barrier (__syncthreads' release fence would wait for them too,
// and the raw bytes of later stages are loaded exactly so that they can).
// The empty asm statements keep the compiler from moving memory accesses
// across it.
__device__ __forceinline__ void lds_barrier() {
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // vmcnt 63, expcnt 7, lgkmcnt 0
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Two E4M3 scale bytes (the low 16 bits) -> an FP16 pair: the packed FP8
// decode is exact, and every E4M3 value is exact in FP16, so the
// round-toward-zero packing does not round.
__device__ __forceinline__ f16x2_t scale_pair(uint32_t two) {
    const f32x2_t f = __builtin_amdgcn_cvt_pk_f32_fp8(static_cast<int>(two), false);
    return __builtin_bit_cast(f16x2_t, __builtin_amdgcn_cvt_pkrtz(f.x, f.y));
}

// Row `row` of a stage tile is 128 bytes, eight 16-byte chunks; chunk c sits
// at c ^ (row & 7) ^ ((row >> 3) & 3). Every wave's fragment reads and
// dequantised stores cover an aligned run of 32 rows, and within one the
// pattern gives rows r, r + 8, r + 16 and r + 24 and any eight consecutive
// rows different chunk positions: measured on gfx950, neither the reads nor
// the 16-byte stores conflict (bank-conflict cycles 366 -> 58 M a call
// against c ^ ((row >> 1) & 7), whose stores took ~8 conflict cycles each).
// The pattern repeats every 32 rows, so the fragment reads of rows 32 apart
// share one address register and differ by an immediate offset (a pattern
// without that period, c ^ ((row ^ (row >> 3)) & 7), also avoided the
// conflicts but ran 7% slower).
__device__ __forceinline__ int chunk_off(int row, int c) {
    return row * 128 + ((c ^ (row & 7) ^ ((row >> 3) & 3)) << 4);
}

// silu(g) = g / (1 + e^-g), through e = e^-|g| so that the exponential never
// overflows: g / (1 + e) for g >= 0, g e / (1 + e) below. FP32 throughout,
// with v_rcp_f32 (1 ulp) for 1 / (1 + e), in [1/2, 1]: a few ulp in all, as
// the IEEE-rounded division was, and 4% faster over the whole kernel.
__device__ __forceinline__ float silu(float g) {
    const float e = expf(-fabsf(g));
    const float r = __builtin_amdgcn_rcpf(1.0f + e);
    return g >= 0.f ? g * r : (g * e) * r;
}

// SWIGLU: the weights hold 2 N_out rows, the gate projection's rows first,
// then the up projection's. In a block's B tile, 32-row tile jt holds the
// gate and up rows of the 16 output columns n0_out + 16 jt + j, j < 16, with
// tile row rr = 8 (j >> 2) + 4 half + (j & 3) (half 0 gate, 1 up): the rows
// one MFMA accumulator gives lanes 0-31 are the gate rows, those it gives
// lanes 32-63 the up rows of the same columns, in the same register.
__device__ __forceinline__ int swiglu_weight_row(int br, int n0_out, int n_out) {
    const int jt = br >> 5, rr = br & 31;
    const int half = (rr >> 2) & 1;
    const int j = ((rr >> 3) << 2) | (rr & 3);
    return half * n_out + n0_out + 16 * jt + j;
}

template <bool SWIGLU, int WM, int WN, int MT, int NT>
__global__ __launch_bounds__(WM * WN * 64) __attribute__((amdgpu_waves_per_eu(2))) void fc1_gemm_kernel(
    const uint8_t* __restrict__ x_packed, const uint8_t* __restrict__ x_scales,
    const float* __restrict__ x_gs, const int32_t* __restrict__ perm, const int32_t* __restrict__ tile_start,
    const int4* __restrict__ tile_info, int k, const uint8_t* __restrict__ w_packed,
    const uint8_t* __restrict__ w_scales, const float* __restrict__ w_gs, const float* __restrict__ y_gs,
    int K, int N, int E, int n_pos, int m_upper, uint8_t* __restrict__ y_packed,
    uint8_t* __restrict__ y_scales) {
    using S = FcShape<WM, WN, MT, NT>;
    constexpr int BM = S::BM, BN = S::BN, NBI = S::NBI;
    extern __shared__ __attribute__((aligned(16))) char lds[];
    const int tid = threadIdx.x, lane = __lane_id(), wave = tid / kWave;
    // Logical tile (row tile over experts, column tile), column tile fastest,
    // split into eight contiguous runs, one per XCD (block b runs on XCD
    // b % 8): an XCD's neighbouring blocks share the gathered A tile, and an
    // expert's weights, in its L2. The runs cover only the row tiles that
    // exist (the grid is sized for the upper bound m_upper).
    const int total = min(tile_start[E], m_upper);
    const int ntn = N / BN;
    const int per = (total * ntn + 7) / 8;
    const int idx = blockIdx.x / 8;
    if (idx >= per) return;
    const int logical = (blockIdx.x % 8) * per + idx;
    const int mt = logical / ntn;
    if (mt >= total) return;
    const int nt = logical - mt * ntn;
    const int4 info = tile_info[mt];
    const int e = info.x, m0 = info.y, row_end = info.z;
    const int n0 = nt * BN;                         // first weight row (Relu2)
    const int n_out = SWIGLU ? N / 2 : N;           // output columns
    const int n0_out = SWIGLU ? nt * (BN / 2) : n0;

    // this thread's load assignment: row r of the A tile, K half h of a
    // stage; B row halves tid + i THREADS (i < NBI) of the 2 BN
    const int r = tid >> 1, h = tid & 1;
    const int p = m0 + r;
    const int slot = p >= 0 && p < row_end ? perm[p] : -1;
    const bool a_ok = slot >= 0 && slot < n_pos;   // a slot outside [0, T k) reads nothing
    const int token = a_ok ? slot / k : 0;
    const size_t kb = static_cast<size_t>(K) / 2, ks = static_cast<size_t>(K) / 16;
    const uint8_t* xa = x_packed + static_cast<size_t>(token) * kb + h * 16;
    const uint8_t* xsrow = x_scales + static_cast<size_t>(token) * ks;
    bool b_ok[NBI];
    int b_r[NBI], b_h[NBI];
    const uint8_t* wb[NBI];
    const uint8_t* wsb[NBI];
#pragma unroll
    for (int i = 0; i < NBI; ++i) {
        const int idx = tid + i * S::THREADS;
        b_ok[i] = idx < 2 * BN;
        b_r[i] = b_ok[i] ? idx >> 1 : 0;
        b_h[i] = idx & 1;
        const int brow = SWIGLU ? swiglu_weight_row(b_r[i], n0_out, n_out) : n0 + b_r[i];
        const size_t wrow = static_cast<size_t>(e) * N + brow;
        wb[i] = w_packed + wrow * kb + b_h[i] * 16;
        wsb[i] = w_scales + wrow * ks;
    }

    // Raw FP4 bytes of one stage (registers) and its scale bytes (LDS).
    // Loads always read a valid row (token 0 for a missing row, the last
    // stage past the end), so they carry no branches; a missing row gets
    // zero scales.
    struct Raw {
        u32x4 a, b[NBI];
        f16x2_t sa, sb[NBI];   // the stage's two scales of each row half, decoded
    };
    const int nst = K / kFcKS;
    auto load_raw = [&](int st, Raw& R) {
        const int kk = (st < nst ? st : nst - 1) * kFcKS;
        R.a = *reinterpret_cast<const u32x4*>(xa + kk / 2);
#pragma unroll
        for (int i = 0; i < NBI; ++i) R.b[i] = *reinterpret_cast<const u32x4*>(wb[i] + kk / 2);
    };
    // Scale bytes go through LDS in chunks of kFcSch stages (32 bytes of a
    // row, loaded as 16 bytes by each of its two threads), double-buffered:
    // one 16-byte request per row half per chunk instead of a 2-byte request
    // per stage, which left most of every L2 request unused.
    char* scl = lds + 2 * S::STAGE;
    const int ksb = K / 16;                 // scale bytes per row (a multiple of 4)
    struct Scl {
        uint32_t a[4], b[NBI][4];
    };
    auto load_scl = [&](int c, Scl& X) {
        const int oa = c * (kFcSch * 4) + 16 * h;
#pragma unroll
        for (int d = 0; d < 4; ++d)
            X.a[d] = oa + 4 * d < ksb ? *reinterpret_cast<const uint32_t*>(xsrow + oa + 4 * d) : 0u;
#pragma unroll
        for (int i = 0; i < NBI; ++i) {
            const int ob = c * (kFcSch * 4) + 16 * b_h[i];
#pragma unroll
            for (int d = 0; d < 4; ++d)
                X.b[i][d] = ob + 4 * d < ksb ? *reinterpret_cast<const uint32_t*>(wsb[i] + ob + 4 * d) : 0u;
        }
    };
    auto write_scl = [&](int c, const Scl& X) {
        char* base = scl + (c & 1) * S::SCHUNK;
        *reinterpret_cast<u32x4*>(base + r * 32 + 16 * h) =
            a_ok ? u32x4{X.a[0], X.a[1], X.a[2], X.a[3]} : u32x4{0u, 0u, 0u, 0u};
#pragma unroll
        for (int i = 0; i < NBI; ++i)
            if (b_ok[i])
                *reinterpret_cast<u32x4*>(base + (BM + b_r[i]) * 32 + 16 * b_h[i]) =
                    u32x4{X.b[i][0], X.b[i][1], X.b[i][2], X.b[i][3]};
    };
    // this thread's two scales of stage st (its K half), decoded once
    auto read_scl = [&](int st, Raw& R) {
        const char* base = scl + ((st / kFcSch) & 1) * S::SCHUNK + 4 * (st % kFcSch);
        R.sa = scale_pair(*reinterpret_cast<const uint16_t*>(base + r * 32 + 2 * h));
#pragma unroll
        for (int i = 0; i < NBI; ++i)
            R.sb[i] = scale_pair(*reinterpret_cast<const uint16_t*>(base + (BM + b_r[i]) * 32 + 2 * b_h[i]));
    };
    // Word q of the stage's 16 bytes (8 elements, scale byte q / 2) of each
    // of this thread's row halves, dequantised into 16-byte chunk 4 h + q of
    // its row in buffer `buf`.
    auto store_word = [&](const Raw& R, int q, int buf) {
        char* A = lds + buf * S::STAGE;
        char* B = A + BM * kFcKS * 2;
        const uint32_t wa = q == 0 ? R.a.x : q == 1 ? R.a.y : q == 2 ? R.a.z : R.a.w;
        const _Float16 sA = q < 2 ? R.sa.x : R.sa.y;
        uint32_t d[4];
        dequant8(wa, f16x2_t{sA, sA}, d);
        *reinterpret_cast<u32x4*>(A + chunk_off(r, 4 * h + q)) = u32x4{d[0], d[1], d[2], d[3]};
#pragma unroll
        for (int i = 0; i < NBI; ++i) {
            if (b_ok[i]) {
                const u32x4 rb = R.b[i];
                const uint32_t wbw = q == 0 ? rb.x : q == 1 ? rb.y : q == 2 ? rb.z : rb.w;
                const _Float16 sB = q < 2 ? R.sb[i].x : R.sb[i].y;
                dequant8(wbw, f16x2_t{sB, sB}, d);
                *reinterpret_cast<u32x4*>(B + chunk_off(b_r[i], 4 * b_h[i] + q)) = u32x4{d[0], d[1], d[2], d[3]};
            }
        }
    };

    f32x16_t acc[MT][NT];
#pragma unroll
    for (int i = 0; i < MT; ++i)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int q = 0; q < 16; ++q) acc[i][j][q] = 0.f;
    const int wm = wave / WN, wn = wave % WN;
    const int frow = lane & 31, hc = lane >> 5;

    // Stage s: the MFMAs on buffer s % 2 are interleaved with the
    // dequantisation of stage s + 1 into the other buffer; the raw bytes of
    // stage s + kFcRaw are loaded at the start of stage s, so a load has
    // kFcRaw - 1 stages to arrive.
    // Scale chunk c + 1 is loaded at stage kFcSch c (chunk 1 here) and
    // written to LDS at stage kFcSch c + kFcSch / 2, into the buffer chunk
    // c - 1 left (its last read was at stage kFcSch c - 2); it is first read
    // at stage kFcSch (c + 1) - 1.
    Raw raw[kFcRaw];
    Scl sc;
#pragma unroll
    for (int i = 0; i < kFcRaw; ++i) load_raw(i, raw[i]);
    load_scl(0, sc);
    write_scl(0, sc);
    if (kFcSch < nst) load_scl(1, sc);
    lds_barrier();
    read_scl(0, raw[0]);
#pragma unroll
    for (int q = 0; q < 4; ++q) store_word(raw[0], q, 0);
    lds_barrier();
    auto stage = [&](int st, Raw& cur, Raw& nxt) {
        load_raw(st + kFcRaw, cur);       // cur's bytes were dequantised during stage st - 1
        const int c = st / kFcSch, u = st % kFcSch;
        if ((c + 1) * kFcSch < nst) {
            if (u == 0 && c > 0) load_scl(c + 1, sc);
            if (u == kFcSch / 2) write_scl(c + 1, sc);
        }
        if (st + 1 < nst) read_scl(st + 1, nxt);
        const char* A = lds + (st & 1) * S::STAGE;
        const char* B = A + BM * kFcKS * 2;
#pragma unroll
        for (int j = 0; j < kFcKS / 16; ++j) {
            f16x8_t a[MT], b[NT];
#pragma unroll
            for (int i = 0; i < MT; ++i)
                a[i] = *reinterpret_cast<const f16x8_t*>(A + chunk_off(wm * 32 * MT + i * 32 + frow, 2 * j + hc));
#pragma unroll
            for (int i = 0; i < NT; ++i)
                b[i] = *reinterpret_cast<const f16x8_t*>(B + chunk_off(wn * 32 * NT + i * 32 + frow, 2 * j + hc));
#pragma unroll
            for (int i = 0; i < MT; ++i)
#pragma unroll
                for (int jn = 0; jn < NT; ++jn)
                    acc[i][jn] = __builtin_amdgcn_mfma_f32_32x32x16_f16(b[jn], a[i], acc[i][jn], 0, 0, 0);
            if (st + 1 < nst) store_word(nxt, j, (st + 1) & 1);
        }
        lds_barrier();
    };
    // whole rounds of kFcRaw stages carry no conditions, so the compiler can
    // count the loads in flight exactly (and waits only for the oldest);
    // the remaining nst % kFcRaw stages follow
    int s0 = 0;
    for (; s0 + kFcRaw <= nst; s0 += kFcRaw) {
#pragma unroll
        for (int u = 0; u < kFcRaw; ++u) stage(s0 + u, raw[u], raw[(u + 1) % kFcRaw]);
    }
#pragma unroll
    for (int u = 0; u < kFcRaw - 1; ++u)
        if (s0 + u < nst) stage(s0 + u, raw[u], raw[(u + 1) % kFcRaw]);

    // Epilogue, from the accumulators (no LDS): the MFMAs ran with the weight
    // rows as the first operand, so lane l of accumulator (i, jn) holds
    // grouped row (l & 31) of row tile i and weight rows 8 (q >> 2) +
    // 4 (l >> 5) + (q & 3), q < 16, of column tile jn.
    //  Relu2: a 16-column output block is values q = 8 blk .. 8 blk + 7 of
    //  lanes l and l + 32, which meet through one v_permlane32_swap for the
    //  block maximum and one for the codes.
    //  SwiGLU: lane l < 32 holds the gate values of the tile's 16 columns,
    //  lane l + 32 the up values (q = column); one swap per pair (q, q + 8)
    //  gives the lower lane gate and up of columns 0-7, the upper lane those
    //  of columns 8-15, so each lane encodes 8 codes of the block and writes
    //  them itself, and only the block maximum crosses lanes.
    // Then the pre-expert quantiser's FP32 steps.
    const float alpha = 1.0f / (*x_gs * w_gs[e]);
    const float gs = *y_gs;
    const float rcp_gs = 1.0f / gs;
    constexpr float kRcp6 = 1.0f / 6.0f;
    const size_t yrow_b = static_cast<size_t>(n_out) / 2, yrow_s = static_cast<size_t>(n_out) / 16;
    const int half = lane >> 5;
    // E4M3 scale byte and the 8 codes of y under it (q = y out, -0 -> +0)
    auto encode8 = [&](const float (&y)[8], float amax, uint32_t& sf, uint32_t& w) {
        const float sc = gs * (amax * kRcp6);
        sf = e4m3_scale_code(sc);
        const float sf_f = __builtin_amdgcn_cvt_f32_fp8(static_cast<int>(sf), 0);
        const float d = sf_f * rcp_gs;
        const float outs = (sf_f != 0.f) ? 1.0f / d : 0.f;
        w = 0;
        if (amax < INFINITY && fabsf(outs) < INFINITY) {
            // the hardware conversion with unit scale rounds finite values to
            // nearest even and saturates
            float q[8];
#pragma unroll
            for (int u = 0; u < 8; ++u) q[u] = __builtin_fmaf(y[u], outs, 0.0f);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[0], q[1], 1.0f, 0);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[2], q[3], 1.0f, 1);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[4], q[5], 1.0f, 2);
            w = __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(w, q[6], q[7], 1.0f, 3);
        } else {
#pragma unroll
            for (int u = 0; u < 8; ++u) w |= e2m1_code(y[u] * outs) << (4 * u);
        }
    };
    auto pair_max = [](float lm) {
        const auto mx = __builtin_amdgcn_permlane32_swap(__float_as_uint(lm), __float_as_uint(lm), false, false);
        return fmaxf(__uint_as_float(mx[0]), __uint_as_float(mx[1]));
    };
    // Relu2: lane pair (l, l + 32) -> the block's 8 code bytes: the lower lane
    // writes bytes 0-3 (its codes 0-3, the upper lane's 4-7), the upper lane
    // bytes 4-7 (its codes 12-15 after the lower lane's 8-11)
    const uint32_t sel = half ? 0x07060302u : 0x05040100u;
#pragma unroll
    for (int i = 0; i < MT; ++i) {
        const int pr = m0 + wm * 32 * MT + i * 32 + (lane & 31);
        const bool row_ok = pr >= 0 && pr < row_end;
#pragma unroll
        for (int jn = 0; jn < NT; ++jn) {
            if constexpr (SWIGLU) {
                const int c0 = n0_out + 16 * (wn * NT + jn);
                float y[8];
                float lm = 0.f;
#pragma unroll
                for (int u = 0; u < 8; ++u) {
                    const auto gu = __builtin_amdgcn_permlane32_swap(__float_as_uint(acc[i][jn][u]),
                                                                     __float_as_uint(acc[i][jn][8 + u]), false, false);
                    const float g = alpha * __uint_as_float(gu[0]);
                    const float v = alpha * __uint_as_float(gu[1]);
                    y[u] = silu(g) * v;
                    lm = fmaxf(lm, fabsf(y[u]));
                }
                uint32_t sf, w;
                encode8(y, pair_max(lm), sf, w);
                if (row_ok) {
                    *reinterpret_cast<uint32_t*>(y_packed + static_cast<size_t>(pr) * yrow_b + c0 / 2 + 4 * half) = w;
                    if (half == 0) y_scales[static_cast<size_t>(pr) * yrow_s + c0 / 16] = static_cast<uint8_t>(sf);
                }
            } else {
                const int c0 = n0 + wn * 32 * NT + jn * 32;
#pragma unroll
                for (int blk = 0; blk < 2; ++blk) {
                    float y[8];
#pragma unroll
                    for (int u = 0; u < 8; ++u) {
                        const float v = alpha * acc[i][jn][8 * blk + u];
                        const float rl = v > 0.f ? v : 0.f;
                        y[u] = rl * rl;
                    }
                    const float lm = fmaxf(fmaxf(fmaxf(y[0], y[1]), fmaxf(y[2], y[3])),
                                           fmaxf(fmaxf(y[4], y[5]), fmaxf(y[6], y[7])));
                    uint32_t sf, w;
                    encode8(y, pair_max(lm), sf, w);                    // y >= 0
                    const auto ws = __builtin_amdgcn_permlane32_swap(w, w, false, false);
                    const uint32_t word = __builtin_amdgcn_perm(ws[1], ws[0], sel);
                    if (row_ok) {
                        const int cb = c0 + 16 * blk;
                        *reinterpret_cast<uint32_t*>(y_packed + static_cast<size_t>(pr) * yrow_b + cb / 2 + 4 * half) = word;
                        if (half == 0) y_scales[static_cast<size_t>(pr) * yrow_s + cb / 16] = static_cast<uint8_t>(sf);
                    }
                }
            }
        }
    }
}

// Smallest row tile of any configuration: sizes the workspace's tile table.
constexpr int kFcMinBM = 128;

// Lays out the row tiles of this configuration's height, then launches the
// GEMM over them.
template <bool SWIGLU, int WM, int WN, int MT, int NT>
int launch_fc1(const uint8_t* x_packed, const uint8_t* x_scales, const float* x_gs, const int32_t* perm,
               const int32_t* offsets, int32_t* tile_start, int4* tile_info, int k, const uint8_t* w_packed,
               const uint8_t* w_scales, const float* w_gs, const float* y_gs, int K, int N, int E,
               long long P, uint8_t* y_packed, uint8_t* y_scales, void* stream) {
    using S = FcShape<WM, WN, MT, NT>;
    static_assert(S::BM >= kFcMinBM, "the workspace holds tiles of at least kFcMinBM rows");
    const long long m_upper = fc1_row_tiles_upper(P, E, S::BM);
    const long long tiles = m_upper * (N / S::BN);
    const long long per_xcd = (tiles + 7) / 8;
    if (per_xcd * 8 >= (1ll << 31)) return MOE_ERR_BAD_SHAPE;
    const int rc = launch(fc1_tiles_kernel, dim3(1), dim3(kFcTilesBlock), 0, stream, offsets, E,
                          static_cast<int>(P), S::BM, static_cast<int>(m_upper), tile_start, tile_info);
    if (rc) return rc;
    return launch(fc1_gemm_kernel<SWIGLU, WM, WN, MT, NT>, dim3(static_cast<unsigned>(per_xcd * 8)), dim3(S::THREADS),
                  S::LDS, stream, x_packed, x_scales, x_gs, perm, tile_start, tile_info, k, w_packed,
                  w_scales, w_gs, y_gs, K, N, E, static_cast<int>(P), static_cast<int>(m_upper),
                  y_packed, y_scales);
}

}  // namespace
}  // namespace moe

namespace moe {
namespace {
// Workspace: tile_start [E + 1] int32, padded to 256 bytes, then tile_info
// [fc1_row_tiles_upper] int4.
size_t fc1_tile_start_bytes(int E) { return (static_cast<size_t>(E + 1) * sizeof(int32_t) + 255) / 256 * 256; }
}  // namespace
}  // namespace moe

extern "C" size_t moe_expert_fc1_workspace_bytes(int T, int k, int E) {
    using namespace moe;
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return 0;
    const long long P = static_cast<long long>(T) * k;
    if (P >= (1ll << 31)) return 0;
    return fc1_tile_start_bytes(E) + static_cast<size_t>(fc1_row_tiles_upper(P, E, kFcMinBM)) * sizeof(int4);
}

namespace moe {
namespace {
// Shared argument checks, zero fill of the unrouted rows and launch. N is
// the output width; the weights hold N rows (Relu2) or 2 N (SwiGLU).
template <bool SWIGLU>
int expert_fc1(const uint8_t* x_packed, const uint8_t* x_scales, const float* x_global_scale,
               const int32_t* perm, const int32_t* offsets, int T, int k, const uint8_t* w_packed,
               const uint8_t* w_scales, const float* w_global_scale, const float* y_global_scale, int K,
               int N, int E, uint8_t* y_packed, uint8_t* y_scales, void* workspace,
               size_t workspace_bytes, void* stream) {
    if (T < 0 || k < 1 || k > MOE_MAX_TOPK || E < 1 || E > MOE_MAX_EXPERTS) return MOE_ERR_BAD_SHAPE;
    const bool n_ok = SWIGLU ? (N >= 64 && N % 64 == 0) : (N >= 128 && N % 128 == 0);
    if (K < kFcKS || K > MOE_MAX_HIDDEN || K % kFcKS != 0 || !n_ok || N > 8 * MOE_MAX_HIDDEN)
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
    const size_t need = moe_expert_fc1_workspace_bytes(T, k, E);
    if (!workspace || workspace_bytes < need) return MOE_ERR_WORKSPACE;
    if (!aligned16(workspace)) return MOE_ERR_ALIGN;
    int32_t* tile_start = static_cast<int32_t*>(workspace);
    int4* tile_info = reinterpret_cast<int4*>(static_cast<char*>(workspace) + fc1_tile_start_bytes(E));

    const int cap = device_cu_count() * 8;
    const long long fill_vec = P * (N / 32);
    const int gf = static_cast<int>(fill_vec / 256 + 1 < cap ? fill_vec / 256 + 1 : cap);
    const int rc = launch(fc1_fill_kernel, dim3(gf), dim3(256), 0, stream, offsets, E, static_cast<int>(P), N,
                reinterpret_cast<u32x4*>(y_packed), reinterpret_cast<uint32_t*>(y_scales));
    if (rc) return rc;
    // widest column tile that divides the weight rows: 192, 256 or 128 rows
    // (96, 128 or 64 output columns under SwiGLU); with fewer than 1024
    // routed rows an expert on average, 128 x 128 tiles of four waves, whose
    // padding is half as much (8192 tokens of top-22 over 512 experts, 352
    // rows each: Relu2 1.67 -> 1.63 ms, SwiGLU 1.74 -> 1.67 ms; from 1408
    // rows the 256-row tiles stay as fast)
    const int rows = SWIGLU ? 2 * N : N;
#define FC1_ARGS x_packed, x_scales, x_global_scale, perm, offsets, tile_start, tile_info, k, w_packed, \
                 w_scales, w_global_scale, y_global_scale, K, rows, E, P, y_packed, y_scales, stream
    if (rows % 128 == 0 && P < 1024ll * E) return launch_fc1<SWIGLU, 2, 2, 2, 2>(FC1_ARGS);
    if (rows % 192 == 0) return launch_fc1<SWIGLU, 4, 2, 2, 3>(FC1_ARGS);
    if (rows % 256 == 0) return launch_fc1<SWIGLU, 2, 4, 4, 2>(FC1_ARGS);
    return launch_fc1<SWIGLU, 4, 2, 2, 2>(FC1_ARGS);
#undef FC1_ARGS
}
}  // namespace
}  // namespace moe

extern "C" int moe_expert_fc1_nvfp4(const uint8_t* x_packed, const uint8_t* x_scales,
                                    const float* x_global_scale, const int32_t* perm,
                                    const int32_t* offsets, int T, int k, const uint8_t* w_packed,
                                    const uint8_t* w_scales, const float* w_global_scale,
                                    const float* y_global_scale, int K, int N, int E,
                                    uint8_t* y_packed, uint8_t* y_scales, void* workspace,
                                    size_t workspace_bytes, void* stream) {
    return moe::expert_fc1<false>(x_packed, x_scales, x_global_scale, perm, offsets, T, k, w_packed, w_scales,
                                  w_global_scale, y_global_scale, K, N, E, y_packed, y_scales, workspace,
                                  workspace_bytes, stream);
}

extern "C" int moe_expert_fc1_swiglu_nvfp4(const uint8_t* x_packed, const uint8_t* x_scales,
                                           const float* x_global_scale, const int32_t* perm,
                                           const int32_t* offsets, int T, int k, const uint8_t* w_packed,
                                           const uint8_t* w_scales, const float* w_global_scale,
                                           const float* y_global_scale, int K, int N, int E,
                                           uint8_t* y_packed, uint8_t* y_scales, void* workspace,
                                           size_t workspace_bytes, void* stream) {
    return moe::expert_fc1<true>(x_packed, x_scales, x_global_scale, perm, offsets, T, k, w_packed, w_scales,
                                 w_global_scale, y_global_scale, K, N, E, y_packed, y_scales, workspace,
                                 workspace_bytes, stream);
}
