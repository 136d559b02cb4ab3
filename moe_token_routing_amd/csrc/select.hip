// Routing selection of moe_route: sigmoid + bias keys, sorted top-k with
// lowest-id ties, renormalised weights, per-token validity mask.
//
// Method: TensorRT-LLM PR #21356 ("Add the Muse Spark Open decoder fast
// paths"), description, Triton kernel "Routing" (sigmoid, bias, top-k,
// renormalised weights; picks sorted by key, an exact tie goes to the lowest
// expert id); lmdeploy PR #4835, MoE gate v2 (required validity mask: an
// invalid token produces no routing entry; the aux-loss-free gate uses the
// bias only to select).
//
// Design (gfx950): one wave per token (for small batches, whose projection
// splits K many ways, four waves sum a token's partials and the first goes
// on alone). For E <= 512 the experts of a lane are
// consecutive (lane e / EPL), so logits and split partials arrive as 16-byte
// vector loads; beyond that expert e lives in lane e % 64 of an LDS copy. The
// sigmoid is evaluated in FP64 and rounded once to FP32 (a correctly rounded
// FP32 sigmoid), the bias added in FP32, and the key mapped to an unsigned
// integer that orders like the float. For small k, each of k rounds takes a
// wave-wide maximum of the lanes' best remaining keys and then, among the
// lanes holding that key, the minimum expert id (both DPP reductions); the
// owner retires its entry. For larger k (E <= 512), the k-th largest key is
// found by a bitwise search with ballot counts, the keys above it and the
// lowest-id keys equal to it are the picks, and each pick's place is its
// rank by (key, id). The sigmoid of the k winners is recomputed from their logits for
// the weights, summed in pick order in FP32 and divided once.
// E <= 512: keys in registers. Larger E: logits staged per wave in LDS.
// The exact FP64 sigmoid is first avoided: approximate keys from the FP32
// hardware exp and reciprocal select a provable superset of the picks
// (filter_select; the k-th largest of the lanes' maxima bounds the cut), and
// only those few get exact keys and are ranked; the exact selection above
// runs only when that superset has more than 64 members (mass ties) or the
// keys are not finite. The kernel is bound by VALU issue (a wave64 op holds a
// 16-lane SIMD for four cycles), which this cuts by about three times. Every
// global load of a token (split partials, biases) is issued before its
// first store, so no wait for loads also waits for stores.
#include <cmath>

#include "launch.hpp"
#include "select.hpp"

namespace moe {
namespace {

constexpr int kSelectBlock = 256;   // four tokens per block, one per wave
constexpr int kSelectWaves = kSelectBlock / kWave;
constexpr int kMaxPicks = MOE_MAX_TOPK;
// From this many picks the k-th largest key is searched bit by bit (about 25
// dependent steps whatever k is) instead of taking k maximum rounds:
// measured at 512 experts, top-22: route 235 -> 211 us; at top-6 and top-8
// the rounds stay faster by 1-4 us.
constexpr int kThresholdPicks = 12;
// Keys first through the FP32 hardware sigmoid (exact FP64 sigmoid only for
// the few candidates that can be among the picks); see filter_select.
#ifndef MOE_SELECT_FILTER
#define MOE_SELECT_FILTER 1
#endif
constexpr bool kSelectFilter = MOE_SELECT_FILTER;


// Monotone map of FP32 keys to unsigned integers; -0 counts as +0 and NaN
// maps to 0, below every number. (A lane with no candidate left is tracked
// by its own flag, not by a key value.)
__device__ __forceinline__ uint32_t ordered_key(float key) {
    uint32_t u = __float_as_uint(key);
    if (u == 0x80000000u) u = 0u;
    if ((u & 0x7FFFFFFFu) > 0x7F800000u) return 0u;
    return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}

// sigmoid(l) evaluated in FP64 and rounded once to FP32
__device__ __forceinline__ float sigmoid_rn(float l) {
    return static_cast<float>(1.0 / (1.0 + exp(-static_cast<double>(l))));
}

constexpr int kSplitBatch = 8;   // split partials loaded before they are added
constexpr int kLdsBatch = 8;   // a lane's experts loaded (or scanned) at once by select_lds_kernel

// value of lane `src` (wave-uniform) of v: v_readlane_b32, no LDS round trip
__device__ __forceinline__ float lane_value(float v, int src) {
    return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), src));
}

// One round's winner given this lane's best remaining candidate (has, bk, be):
// the largest key, and among equal keys the lowest expert id.
__device__ __forceinline__ uint32_t round_winner(bool has, uint32_t bk, uint32_t be) {
    const uint32_t kmax = __reduce_max_sync(~0ull, has ? bk : 0u);
    return __reduce_min_sync(~0ull, (has && bk == kmax) ? be : 0xFFFFFFFFu);
}

// The k-th largest of the wave's live keys (the largest v with at least k
// live keys >= v), found bit by bit from the top: each step counts with one
// ballot per register slot, and the count and the bound stay scalar. Every
// key shares the bits above the highest bit where the smallest and the
// largest key differ, so the search starts below it.
// With coarse = true the search stops at the bit whose step, at the keys'
// magnitude, is 2^-16 or less: the result is then a lower bound of the k-th
// largest key within 2^-15 of it (what filter_select needs).
template <int EPL, bool COARSE = false>
__device__ __forceinline__ uint32_t kth_largest(const uint32_t (&key)[EPL], uint32_t live, int k) {
    uint32_t lo_key = 0xFFFFFFFFu, hi_key = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if ((live >> i) & 1u) {
            lo_key = key[i] < lo_key ? key[i] : lo_key;
            hi_key = key[i] > hi_key ? key[i] : hi_key;
        }
    lo_key = __reduce_min_sync(~0ull, lo_key);
    hi_key = __reduce_max_sync(~0ull, hi_key);
    const uint32_t diff = lo_key ^ hi_key;
    const int top = diff ? 31 - __clz(diff) : -1;   // -1: all keys equal
    uint32_t thr = top < 0 ? lo_key : (top == 31 ? 0u : (lo_key & ~((2u << top) - 1u)));
    int last = 0;
    if constexpr (COARSE) {
        // one step of bit b spans 2^(b + e - 23) at binary exponent e, so
        // with e the largest exponent among the keys, bits below 7 - e are
        // finer than 2^-16 and left at zero (thr only decreases)
        const uint32_t ehi = ((hi_key & 0x80000000u ? hi_key : ~hi_key) >> 23) & 0xFFu;
        const uint32_t elo = ((lo_key & 0x80000000u ? lo_key : ~lo_key) >> 23) & 0xFFu;
        const int e = static_cast<int>(ehi > elo ? ehi : elo) - 127;
        last = min(31, max(0, 7 - e));
        if (top < 0) thr = lo_key & ~((1u << last) - 1u);
    }
#pragma unroll 1
    for (int b = top; b >= last; --b) {
        const uint32_t cand = thr | (1u << b);
        int cnt = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) cnt += __popcll(__ballot(((live >> i) & 1u) && key[i] >= cand));
        if (cnt >= k) thr = cand;
    }
    return thr;
}

// Inverse of ordered_key for the keys of numbers (not 0, which stands for NaN).
__device__ __forceinline__ float key_value(uint32_t o) {
    return __uint_as_float(o & 0x80000000u ? (o & 0x7FFFFFFFu) : ~o);
}

// sigmoid(l) in FP32 hardware approximations, 1 / (1 + 2^(-l log2 e)) with
// v_exp_f32 and v_rcp_f32: its absolute error is below 2^-17 for every l
// (the exponent's argument carries a relative error of 2^-24, so 2^x one of
// |x| ln2 2^-24 < 2^-17.5 while |x| < 128 -- beyond, the sigmoid is within
// 2^-128 of 0 or 1 and so is this -- and the sigmoid's slope is at most 1/4;
// exp and rcp add a few ulp). NaN stays NaN, +-inf give 1 and 0.
__device__ __forceinline__ float sigmoid_approx(float l) {
    const float e = __builtin_amdgcn_exp2f(-l * 1.44269504088896341f);
    return __builtin_amdgcn_rcpf(1.0f + e);
}

// Per-wave LDS of the filtered selection: the candidates (compacted) and the
// picks in order.
struct FilterLds {
    float cand_l[kSelectWaves][kWave];
    float cand_b[kSelectWaves][kWave];   // the candidate's bias (no gather after the logit stores)
    int32_t cand_id[kSelectWaves][kWave];
    int32_t pick_id[kSelectWaves][kMaxPicks];
    float pick_s[kSelectWaves][kMaxPicks];
};

// The C <= 64 candidates in sh.cand_l / cand_b / cand_id (logit, bias and id;
// this wave's rows, in any order): exact keys (FP64 sigmoid rounded once, plus the bias in FP32), each
// ranked among them by (key descending, id ascending); the first k are the
// picks, written with their renormalised weights (sigmoid, FP32 sum in pick
// order, one division). Returns pick `lane`'s id to lane < k.
__device__ __forceinline__ int rank_candidates(int lane, int C, int k, int32_t* __restrict__ ids,
                                               float* __restrict__ w, FilterLds& sh) {
    const int wv = threadIdx.x / kWave;
    // (LDS accesses of one wave complete in order; the fences keep the
    // compiler from moving them across)
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const bool mine = lane < C;
    const float l = mine ? sh.cand_l[wv][lane] : 0.f;
    const int id = mine ? sh.cand_id[wv][lane] : 0;
    const float s = mine ? sigmoid_rn(l) : 0.f;
    const uint32_t key = mine ? ordered_key(s + sh.cand_b[wv][lane]) : 0u;
    int rank = 0;
#pragma unroll 1
    for (int m = 0; m < C; ++m) {
        const uint32_t km = __builtin_amdgcn_readlane(key, m);
        const int im = __builtin_amdgcn_readlane(id, m);
        rank += (km > key || (km == key && im < id)) ? 1 : 0;
    }
    if (mine && rank < k) {
        sh.pick_id[wv][rank] = id;
        sh.pick_s[wv][rank] = s;
    }
    __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
    const float my_s = lane < k ? sh.pick_s[wv][lane] : 0.f;
    const int my_id = lane < k ? sh.pick_id[wv][lane] : -1;
    float total = 0.f;
#pragma unroll 1
    for (int j = 0; j < k; ++j) total += lane_value(my_s, j);
    if (lane < k) {
        ids[lane] = my_id;
        w[lane] = my_s / total;
    }
    return my_id;
}

// Selection of one valid token through approximate keys. A = approx sigmoid +
// bias differs from the exact key K = RN32(RN32(sigmoid) + bias) by at most
// d = 2^-17 + 2^-25 + ulp(K). Let A_k be the k-th largest approximate key:
// the k experts with the largest A have exact keys > A_k - d, so the exact
// k-th largest key is above A_k - d, and every expert of the exact top k has
// A > A_k - 2d. For any lower bound t <= A_k, the experts with A >= t - M
// (M = 2^-15 + max|A| 2^-20 > 2d) are therefore a superset of the top k --
// typically a few more than k. They are compacted one per lane, their exact
// keys computed (FP64 sigmoid rounded once, as everywhere else), and each is
// ranked among them by (key descending, id ascending): the same picks, order
// and weights as the exact selection over all experts. Returns false
// (nothing written) when the bound is NaN or infinite, or fewer than k or
// more than 64 experts pass; the caller then runs the exact selection. Lane
// j < k returns pick j's id in `pick`.
template <int EPL>
__device__ __forceinline__ bool filter_select(int lane, int e0, uint32_t live, const float (&lg)[EPL],
                                              const float (&bs)[EPL], int k, int32_t* __restrict__ ids,
                                              float* __restrict__ w, FilterLds& sh, int& pick) {
    const int wv = threadIdx.x / kWave;
    float A[EPL];
    uint32_t oa[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const bool l = (live >> i) & 1u;
        A[i] = l ? sigmoid_approx(lg[i]) + bs[i] : 0.f;
        oa[i] = l ? ordered_key(A[i]) : 0u;
    }
    // The k-th largest of the lanes' largest approximate keys: k distinct
    // experts lie at or above it, so it is at most A_k (and a coarse lower
    // bound of it serves as well); one key per lane to search instead of all
    // of them (measured: selection at 512 experts, top-22, 32768 tokens 65 ->
    // 49 us). M's relative term is taken at the largest |A| of the row, which
    // covers the ulp of every key however far below A_k the bound lies.
    uint32_t lmax = 0u;
    float labs = 0.f;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if ((live >> i) & 1u) {
            lmax = max(lmax, oa[i]);
            labs = fmaxf(labs, fabsf(A[i]));
        }
    const uint32_t top1[1] = {lmax};
    const uint32_t kth = kth_largest<1, true>(top1, live != 0u ? 1u : 0u, k);
    if (kth == 0u) return false;   // fewer than k lanes hold a number
    // (non-negative values order like their bit patterns)
    const float amax = __uint_as_float(__reduce_max_sync(~0ull, __float_as_uint(labs)));
    const float lo = key_value(kth) - (0x1p-15f + amax * 0x1p-20f);
    uint32_t cand = 0u;
#pragma unroll
    for (int i = 0; i < EPL; ++i) cand |= static_cast<uint32_t>(((live >> i) & 1u) && A[i] >= lo) << i;
    const uint64_t below = lanemask_lt();
    int C = 0, pos = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        const uint64_t b = __ballot((cand >> i) & 1u);
        C += __popcll(b);
        pos += __popcll(b & below);
    }
    // (fewer than k: the cut is NaN, an infinite key; then the exact path)
    if (C < k || C > kWave) return false;
#pragma unroll
    for (int i = 0; i < EPL; ++i)
        if ((cand >> i) & 1u) {
            sh.cand_l[wv][pos] = lg[i];
            sh.cand_b[wv][pos] = bs[i];
            sh.cand_id[wv][pos] = e0 + i;
            ++pos;
        }
    pick = rank_candidates(lane, C, k, ids, w, sh);
    return true;
}


// The k picks' weights: sigmoid of each winner's logit, FP32 sum in pick
// order, one division; lane j < k writes pick j.
__device__ __forceinline__ void write_picks(int lane, int k, int my_id, float my_l,
                                            int32_t* __restrict__ ids, float* __restrict__ w) {
    const float my_s = lane < k ? sigmoid_rn(my_l) : 0.f;
    float total = 0.f;
#pragma unroll 1
    for (int j = 0; j < k; ++j) total += lane_value(my_s, j);
    if (lane < k) {
        ids[lane] = my_id;
        w[lane] = my_s / total;
    }
}

// With `hist` set, lane j < k counts token t's pick j into the expert
// histogram of its tile of dispatch slots: hist[(t k + j) / hist_tile][id]
// += 1 (slot t k + j is pick j of token t, as moe_dispatch numbers them).
// Integer additions commute, so the counts do not depend on the order in
// which waves arrive; the add returns nothing, so the wave does not wait.
__device__ __forceinline__ void count_pick(int32_t* __restrict__ hist, int hist_tile, int E, int t, int k,
                                          int lane, int id) {
    if (hist && lane < k && id >= 0) {
        const long long slot = static_cast<long long>(t) * k + lane;
        __hip_atomic_fetch_add(hist + (slot / hist_tile) * E + id, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
}

// EPL consecutive floats at p (16-byte vector loads when `vec`, which the
// caller sets when the row length keeps them aligned). NT: the full-lane
// 16-byte loads non-temporal (data read once, the projection's split-K
// partials), so that they do not crowd the caches ahead of the next
// kernel's reads: at 8192 tokens the route + dispatch + norm + quant call
// 147.4 -> 143.0 us and the step 365.4 -> 359.8 us (three alternating runs).
typedef float f32x4_t __attribute__((ext_vector_type(4)));
template <int EPL, bool FULL, bool NT = false>
__device__ __forceinline__ void load_run(const float* __restrict__ p, bool vec, int n, float (&v)[EPL]) {
    if constexpr (FULL) {
        // every lane owns EPL experts and rows are 16-byte aligned: plain
        // vector loads, no bounds (the full-lane case is decided per launch)
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                f32x4_t q;
                if constexpr (NT)
                    q = __builtin_nontemporal_load(reinterpret_cast<const f32x4_t*>(p + i));
                else
                    q = *reinterpret_cast<const f32x4_t*>(p + i);
                v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
            }
        } else {
#pragma unroll
            for (int i = 0; i < EPL; ++i) v[i] = p[i];
        }
        return;
    }
    if constexpr (EPL % 4 == 0) {
        if (vec) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const float4 q = *reinterpret_cast<const float4*>(p + i);
                v[i] = q.x; v[i + 1] = q.y; v[i + 2] = q.z; v[i + 3] = q.w;
            }
            return;
        }
    }
#pragma unroll
    for (int i = 0; i < EPL; ++i) v[i] = i < n ? p[i] : 0.f;
}

// Experts e = EPL*lane + i (i < EPL) live in lane e / EPL, so each lane reads
// its logits (or split partials) as one contiguous run. BATCH split partials
// are loaded before any of them is added: 8 keep the registers of many waves
// per SIMD (large batches split K 8 ways).
// WPT waves per token: with WPT = 4 (small batches, whose projection splits
// K many ways: 64 at 128 tokens) a block is one token and its four waves
// each sum a contiguous quarter of the splits, so a token's partials are
// read by one CU's four SIMDs at once (and the batch by four times as many
// CUs); the quarter sums meet in LDS, added in order to the first, and the
// first wave goes on alone.
template <int EPL, int BATCH, bool THRESHOLD, bool FULL, int WPT = 1>
__global__ __launch_bounds__(kSelectBlock) void select_reg_kernel(
    const float* __restrict__ partials, int nsplit, float scale, int logits_in,
    const float* __restrict__ bias, const uint8_t* __restrict__ token_mask, int T, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, int hist_tile) {
    static_assert(WPT == 1 || WPT == kSelectWaves, "one token per wave or per block");
    const int lane = __lane_id();
    const int wq = WPT == 1 ? 0 : static_cast<int>(threadIdx.x) / kWave;   // quarter of the splits
    const int t = WPT == 1 ? blockIdx.x * kSelectWaves + static_cast<int>(threadIdx.x) / kWave
                           : static_cast<int>(blockIdx.x);
    if (t >= T) return;   // whole wave (WPT = 4: whole block) leaves together
    if (WPT > 1 && logits_in && wq > 0) return;   // (not launched so: nothing to sum)
    const size_t plane = static_cast<size_t>(T) * E;
    const bool valid = token_mask[t] != 0;
    const int e0 = EPL * lane;
    // experts of this lane (FULL: E = EPL * 64, every lane owns EPL)
    const int n = FULL ? EPL : (E - e0 < EPL ? (E - e0 > 0 ? E - e0 : 0) : EPL);
    const bool vec = FULL || ((E % 4) == 0 && n == EPL);
    const size_t row = static_cast<size_t>(t) * E + e0;

    float lg[EPL], bs[EPL];
    // the lane's biases, loaded with its logits (before any store)
    if (n > 0 && wq == 0) {
        load_run<EPL, FULL>(bias + e0, vec, n, bs);
    } else {
#pragma unroll
        for (int i = 0; i < EPL; ++i) bs[i] = 0.f;
    }
    // this wave's splits [s0, s1): all of them, or (WPT = 4) a contiguous
    // quarter, every quarter nonempty (nsplit > 9 when WPT = 4)
    const int per = (nsplit + WPT - 1) / WPT;
    const int s0 = wq * per, s1 = min(nsplit, s0 + per);
#pragma unroll
    for (int i = 0; i < EPL; ++i) lg[i] = 0.f;
    if (n > 0) {
        if (logits_in) {
            load_run<EPL, FULL>(logits + row, vec, n, lg);
        } else {
            load_run<EPL, FULL, true>(partials + s0 * plane + row, vec, n, lg);
            // a batch of splits is loaded before any is added (the loads
            // overlap); the sum still runs over the splits in order
#pragma unroll 1
            for (int p0 = s0 + 1; p0 < s1; p0 += BATCH) {
                float q[BATCH][EPL];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    if (p0 + u < s1) {
                        load_run<EPL, FULL, true>(partials + (p0 + u) * plane + row, vec, n, q[u]);
                    } else {
#pragma unroll
                        for (int i = 0; i < EPL; ++i) q[u][i] = 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (p0 + u < s1) {
#pragma unroll
                        for (int i = 0; i < EPL; ++i) lg[i] += q[u][i];
                    }
            }
        }
    }
    if constexpr (WPT > 1) {
        if (!logits_in) {
            // the quarters meet: waves 1..3 hand their sums to wave 0, which
            // adds them in order (uniform control flow around the barrier)
            __shared__ float quarter[WPT - 1][EPL][kWave];
            if (wq > 0) {
#pragma unroll
                for (int i = 0; i < EPL; ++i) quarter[wq - 1][i][lane] = lg[i];
            }
            __syncthreads();
            if (wq > 0) return;
#pragma unroll
            for (int w = 0; w < WPT - 1; ++w)
#pragma unroll
                for (int i = 0; i < EPL; ++i) lg[i] += quarter[w][i][lane];
        }
    }
    if (n > 0 && !logits_in) {
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            lg[i] *= scale;
            if (i < n) logits[row + i] = lg[i];
        }
    }
    int32_t* ids = topk_ids + static_cast<size_t>(t) * k;
    float* w = topk_w + static_cast<size_t>(t) * k;
    if (!valid) {
        for (int j = lane; j < k; j += kWave) {
            ids[j] = -1;
            w[j] = 0.f;
        }
        return;
    }
    // bit i: expert EPL*lane + i still a candidate (full lanes: all of them)
    uint32_t live = 0;
#pragma unroll
    for (int i = 0; i < EPL; ++i) live |= static_cast<uint32_t>(FULL || i < n) << i;
    if constexpr (kSelectFilter) {
        __shared__ FilterLds fsh;
        int pick = -1;
        if (filter_select<EPL>(lane, e0, live, lg, bs, k, ids, w, fsh, pick)) {
            count_pick(hist, hist_tile, E, t, k, lane, pick);
            return;
        }
    }
    // exact keys of every expert
    uint32_t key[EPL];
#pragma unroll
    for (int i = 0; i < EPL; ++i) key[i] = ((live >> i) & 1u) ? ordered_key(sigmoid_rn(lg[i]) + bs[i]) : 0u;

    int my_id = -1;
    float my_l = 0.f;
    if constexpr (!THRESHOLD) {
        // k rounds: the wave-wide largest remaining key, the lowest id among
        // its holders, retired by its owner
#pragma unroll 1
        for (int j = 0; j < k; ++j) {
            uint32_t bk = 0u;
            int bi = -1;
            float bl = 0.f;
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                const bool take = ((live >> i) & 1u) && (bi < 0 || key[i] > bk);
                bk = take ? key[i] : bk;
                bl = take ? lg[i] : bl;
                bi = take ? i : bi;
            }
            const uint32_t win = round_winner(bi >= 0, bk, static_cast<uint32_t>(e0 + bi));
            const int owner = static_cast<int>(win / EPL);
            const float l_win = lane_value(bl, owner);
            if (lane == owner) live &= ~(1u << bi);
            if (lane == j) {
                my_id = static_cast<int>(win);
                my_l = l_win;
            }
        }
    } else {
        const uint32_t thr = kth_largest<EPL>(key, live, k);
        // The picks: every key above it, then the keys equal to it with the
        // lowest expert ids (ids run lane-major, e = EPL lane + i).
        uint32_t gt = 0u, eq = 0u;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            const bool l = (live >> i) & 1u;
            gt |= static_cast<uint32_t>(l && key[i] > thr) << i;
            eq |= static_cast<uint32_t>(l && key[i] == thr) << i;
        }
        const uint64_t below = lanemask_lt();
        int n_gt = 0, eq_before = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) {
            n_gt += __popcll(__ballot((gt >> i) & 1u));
            eq_before += __popcll(__ballot((eq >> i) & 1u) & below);
        }
        uint32_t sel = gt;
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if ((eq >> i) & 1u) {
                if (eq_before < k - n_gt) sel |= 1u << i;
                ++eq_before;
            }
        // The k picks, compacted into the wave's LDS list in id order; lane
        // j < k takes entry j, ranks it by (key descending, id ascending) --
        // larger keys, and equal keys earlier in the list -- and puts it in
        // its place.
        __shared__ uint32_t list_key[kSelectWaves][kMaxPicks];
        __shared__ int32_t list_id[kSelectWaves][kMaxPicks];
        __shared__ float list_l[kSelectWaves][kMaxPicks];
        __shared__ int32_t pick_id[kSelectWaves][kMaxPicks];
        __shared__ float pick_l[kSelectWaves][kMaxPicks];
        const int wv = threadIdx.x / kWave;
        int pos = 0;
#pragma unroll
        for (int i = 0; i < EPL; ++i) pos += __popcll(__ballot((sel >> i) & 1u) & below);
#pragma unroll
        for (int i = 0; i < EPL; ++i)
            if ((sel >> i) & 1u) {
                list_key[wv][pos] = key[i];
                list_id[wv][pos] = e0 + i;
                list_l[wv][pos] = lg[i];
                ++pos;
            }
        // (LDS accesses of one wave complete in order; the fences keep the
        // compiler from moving them across)
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        const uint32_t mk = lane < k ? list_key[wv][lane] : 0u;
        const int mid = lane < k ? list_id[wv][lane] : -1;
        const float ml = lane < k ? list_l[wv][lane] : 0.f;
        int rank = 0;
#pragma unroll 1
        for (int m = 0; m < k; ++m) {
            const uint32_t km = __builtin_amdgcn_readlane(mk, m);
            rank += (km > mk || (km == mk && m < lane)) ? 1 : 0;
        }
        if (lane < k) {
            pick_id[wv][rank] = mid;
            pick_l[wv][rank] = ml;
        }
        __builtin_amdgcn_fence(__ATOMIC_ACQ_REL, "wavefront");
        my_id = lane < k ? pick_id[wv][lane] : -1;
        my_l = lane < k ? pick_l[wv][lane] : 0.f;
    }
    write_picks(lane, k, my_id, my_l, ids, w);
    count_pick(hist, hist_tile, E, t, k, lane, my_id);
}

// Any E: each wave stages its token's logits in its own LDS region (dynamic
// LDS: kSelectWaves * E * 4 bytes). A lane only touches the entries of its
// own experts, so no barrier is needed. The loads of a row (split partials,
// bias) come first, with no stores among them; then the logits are written
// out from LDS. The approximate-key filter (as filter_select, with the k-th
// largest lane maximum as the lower bound) picks the candidates; otherwise
// the exact keys replace the logits in LDS and k rounds pick the experts,
// whose logits are read back from the row. One key per expert in LDS lets
// four blocks share a CU at 2560 experts.
__global__ __launch_bounds__(kSelectBlock) void select_lds_kernel(
    const float* __restrict__ partials, int nsplit, float scale, int logits_in,
    const float* __restrict__ bias, const uint8_t* __restrict__ token_mask, int T, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w,
    int32_t* __restrict__ hist, int hist_tile) {
    extern __shared__ uint32_t sel_lds[];
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kSelectWaves + wave;
    if (t >= T) return;
    uint32_t* keys = sel_lds + static_cast<size_t>(wave) * E;   // the row's logits, later (exact path) its keys
    const size_t plane = static_cast<size_t>(T) * E;
    const bool valid = token_mask[t] != 0;
    const int nloc = lane < E ? (E - lane + kWave - 1) / kWave : 0;   // <= 64
    float* lrow = logits + static_cast<size_t>(t) * E;
    uint32_t lane_top = 0u;   // the lane's largest approximate key (ordered)
    float lane_abs = 0.f;     // and largest magnitude
    // Pass 1, loads only (no store waits between them): the lane's experts
    // e = lane + 64 i, kLdsBatch at a time, their logits (or split partials,
    // split by split) all loaded before any is used; each logit still sums
    // its splits in order. The logits stay in LDS.
#pragma unroll 1
    for (int e0 = lane; e0 < E; e0 += kLdsBatch * kWave) {
        float l[kLdsBatch], b[kLdsBatch];
#pragma unroll
        for (int u = 0; u < kLdsBatch; ++u) {
            const int e = e0 + u * kWave;
            const size_t idx = static_cast<size_t>(t) * E + e;
            l[u] = e < E ? (logits_in ? logits[idx] : partials[idx]) : 0.f;
            b[u] = e < E ? bias[e] : 0.f;
        }
        if (!logits_in) {
#pragma unroll 1
            for (int p = 1; p < nsplit; ++p) {
                float q[kLdsBatch];
#pragma unroll
                for (int u = 0; u < kLdsBatch; ++u) {
                    const int e = e0 + u * kWave;
                    q[u] = e < E ? partials[p * plane + static_cast<size_t>(t) * E + e] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < kLdsBatch; ++u) l[u] += q[u];
            }
#pragma unroll
            for (int u = 0; u < kLdsBatch; ++u) l[u] *= scale;
        }
#pragma unroll
        for (int u = 0; u < kLdsBatch; ++u) {
            const int e = e0 + u * kWave;
            if (e < E) {
                keys[e] = __float_as_uint(l[u]);
                if constexpr (kSelectFilter) {
                    const float a = sigmoid_approx(l[u]) + b[u];
                    lane_top = max(lane_top, ordered_key(a));
                    lane_abs = fmaxf(lane_abs, fabsf(a));
                }
            }
        }
    }
    // Pass 2: the logits row out (stores only)
    if (!logits_in) {
#pragma unroll 1
        for (int i0 = 0; i0 < nloc; i0 += kLdsBatch) {
#pragma unroll
            for (int u = 0; u < kLdsBatch; ++u)
                if (i0 + u < nloc) lrow[lane + kWave * (i0 + u)] = __uint_as_float(keys[lane + kWave * (i0 + u)]);
        }
    }
    int32_t* ids = topk_ids + static_cast<size_t>(t) * k;
    float* w = topk_w + static_cast<size_t>(t) * k;
    if (!valid) {
        for (int j = lane; j < k; j += kWave) {
            ids[j] = -1;
            w[j] = 0.f;
        }
        return;
    }
    if constexpr (kSelectFilter) {
        // The k largest lane maxima are k distinct experts, so the k-th
        // largest of them (a coarse lower bound of it) is at most the k-th
        // largest approximate key A_k; cutting M below it keeps every
        // expert that can be among the exact picks (filter_select's bound,
        // with M's relative term taken at the largest |A| of the row). The
        // scan recomputes each approximate key from the logit in LDS, and a
        // candidate's logit comes from there too.
        __shared__ FilterLds fsh;
        const uint32_t top1[1] = {lane_top};
        const uint32_t kth = kth_largest<1, true>(top1, 1u, k);
        // (non-negative values order like their bit patterns)
        const float amax = __uint_as_float(__reduce_max_sync(~0ull, __float_as_uint(lane_abs)));
        if (kth != 0u) {
            const float kf = key_value(kth);
            const float lo = kf - (0x1p-15f + amax * 0x1p-20f);
            const uint64_t below = lanemask_lt();
            const int wv = threadIdx.x / kWave;
            int C = 0;
            const int nmax = (E + kWave - 1) / kWave;   // slots of lane 0, the most (the ballots need every lane)
#pragma unroll 1
            for (int i0 = 0; i0 < nmax; i0 += kLdsBatch) {
                float lv[kLdsBatch], bv[kLdsBatch];
#pragma unroll
                for (int u = 0; u < kLdsBatch; ++u) {
                    const bool in = i0 + u < nloc;
                    lv[u] = in ? __uint_as_float(keys[lane + kWave * (i0 + u)]) : 0.f;
                    bv[u] = in ? bias[lane + kWave * (i0 + u)] : 0.f;
                }
#pragma unroll
                for (int u = 0; u < kLdsBatch; ++u) {
                    const bool c = i0 + u < nloc && sigmoid_approx(lv[u]) + bv[u] >= lo;
                    const uint64_t bb = __ballot(c);
                    const int pos = C + __popcll(bb & below);
                    if (c && pos < kWave) {
                        fsh.cand_l[wv][pos] = lv[u];
                        fsh.cand_b[wv][pos] = bv[u];
                        fsh.cand_id[wv][pos] = lane + kWave * (i0 + u);
                    }
                    C += __popcll(bb);
                }
            }
            if (C >= k && C <= kWave) {
                const int pick = rank_candidates(lane, C, k, ids, w, fsh);
                count_pick(hist, hist_tile, E, t, k, lane, pick);
                return;
            }
        }
    }
    // the exact keys of every expert (in place of its logit), then the rounds
#pragma unroll 1
    for (int i = 0; i < nloc; ++i) {
        const int e = lane + kWave * i;
        keys[e] = ordered_key(sigmoid_rn(__uint_as_float(keys[e])) + bias[e]);
    }
    uint64_t live = nloc >= 64 ? ~0ull : ((1ull << nloc) - 1);

    int my_id = -1;
#pragma unroll 1
    for (int j = 0; j < k; ++j) {
        uint32_t bk = 0u;
        int bi = -1;
        // the lane's keys in slot order, kLdsBatch LDS reads in flight at a
        // time; a strictly larger key replaces the best, so among equal keys
        // the lowest slot (lowest id) stays
#pragma unroll 1
        for (int i0 = 0; i0 < nloc; i0 += kLdsBatch) {
            uint32_t kv[kLdsBatch];
#pragma unroll
            for (int u = 0; u < kLdsBatch; ++u) kv[u] = i0 + u < nloc ? keys[lane + kWave * (i0 + u)] : 0u;
#pragma unroll
            for (int u = 0; u < kLdsBatch; ++u) {
                const int i = i0 + u;
                const bool take = i < nloc && ((live >> i) & 1ull) && (bi < 0 || kv[u] > bk);
                bk = take ? kv[u] : bk;
                bi = take ? i : bi;
            }
        }
        const uint32_t win = round_winner(bi >= 0, bk, static_cast<uint32_t>(lane + kWave * bi));
        const int owner = static_cast<int>(win & (kWave - 1));
        if (lane == owner) live &= ~(1ull << (win / kWave));
        if (lane == j) my_id = static_cast<int>(win);
    }
    // lane j < k reads pick j's logit from the row (pass 2 wrote it, by the
    // lane that owns the expert: the wave's stores are made visible first)
    __threadfence_block();
    const float my_l = lane < k ? lrow[my_id] : 0.f;
    write_picks(lane, k, my_id, my_l, ids, w);
    count_pick(hist, hist_tile, E, t, k, lane, my_id);
}

template <int EPL, int BATCH, int WPT = 1>
int launch_select_reg2(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
                       const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
                       int32_t* hist, int hist_tile, void* stream) {
    const dim3 grid(ceil_div(T, kSelectWaves / WPT));
#define MOE_SELECT(THR, FULL)                                                                                 \
    return launch(select_reg_kernel<EPL, BATCH, THR, FULL, WPT>, grid, dim3(kSelectBlock), 0, stream, partials,  \
                  nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile)
    const bool full = E == EPL * kWave;   // then E % 4 == 0 and every row is 16-byte aligned
    if (k >= kThresholdPicks) {
        if (full) MOE_SELECT(true, true);
        MOE_SELECT(true, false);
    }
    if (full) MOE_SELECT(false, true);
    MOE_SELECT(false, false);
#undef MOE_SELECT
}

template <int EPL>
int launch_select_reg(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
                      const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
                      int32_t* hist, int hist_tile, void* stream) {
    // many splits (a small batch): four waves per token, each summing a
    // quarter of the splits, up to 16 loads in flight per lane (8 with 8
    // experts a lane, for its registers)
    if (nsplit > 2 * kSplitBatch && !logits_in)
        return launch_select_reg2<EPL, (EPL <= 4 ? 2 : 1) * kSplitBatch, kSelectWaves>(
            partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile, stream);
    return launch_select_reg2<EPL, kSplitBatch>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits,
                                                ids, w, hist, hist_tile, stream);
}

}  // namespace

int run_select(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
               const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
               int32_t* hist, int hist_tile, void* stream) {
    const int epl = ceil_div(E, kWave);
    if (epl <= 1) return launch_select_reg<1>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile, stream);
    if (epl <= 2) return launch_select_reg<2>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile, stream);
    if (epl <= 4) return launch_select_reg<4>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile, stream);
    if (epl <= 8) return launch_select_reg<8>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile, stream);
    const size_t lds = static_cast<size_t>(kSelectWaves) * E * sizeof(uint32_t);
    return launch(select_lds_kernel, dim3(ceil_div(T, kSelectWaves)), dim3(kSelectBlock), lds, stream,
                  partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, hist, hist_tile);
}

}  // namespace moe
