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
// Design (gfx950): one wave per token. For E <= 512 the experts of a lane are
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
// E <= 512: keys in registers. Larger E: keys and logits staged per wave in LDS.
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
constexpr int kLdsBatch = 8;     // a lane's experts loaded (or scanned) at once by select_lds_kernel

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

// EPL consecutive floats at p (16-byte vector loads when `vec`, which the
// caller sets when the row length keeps them aligned).
template <int EPL, bool FULL>
__device__ __forceinline__ void load_run(const float* __restrict__ p, bool vec, int n, float (&v)[EPL]) {
    if constexpr (FULL) {
        // every lane owns EPL experts and rows are 16-byte aligned: plain
        // vector loads, no bounds (the full-lane case is decided per launch)
        if constexpr (EPL % 4 == 0) {
#pragma unroll
            for (int i = 0; i < EPL; i += 4) {
                const float4 q = *reinterpret_cast<const float4*>(p + i);
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
// per SIMD (large batches split K 8 ways); 32 cut the dependent rounds of
// loads when a small batch split K many ways (64 at 128 tokens).
template <int EPL, int BATCH, bool THRESHOLD, bool FULL>
__global__ __launch_bounds__(kSelectBlock) void select_reg_kernel(
    const float* __restrict__ partials, int nsplit, float scale, int logits_in,
    const float* __restrict__ bias, const uint8_t* __restrict__ token_mask, int T, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
    const int lane = __lane_id();
    const int t = blockIdx.x * kSelectWaves + threadIdx.x / kWave;
    if (t >= T) return;   // whole wave leaves together
    const size_t plane = static_cast<size_t>(T) * E;
    const bool valid = token_mask[t] != 0;
    const int e0 = EPL * lane;
    // experts of this lane (FULL: E = EPL * 64, every lane owns EPL)
    const int n = FULL ? EPL : (E - e0 < EPL ? (E - e0 > 0 ? E - e0 : 0) : EPL);
    const bool vec = FULL || ((E % 4) == 0 && n == EPL);
    const size_t row = static_cast<size_t>(t) * E + e0;

    float lg[EPL];
    if (n > 0) {
        if (logits_in) {
            load_run<EPL, FULL>(logits + row, vec, n, lg);
        } else {
            load_run<EPL, FULL>(partials + row, vec, n, lg);
            // a batch of splits is loaded before any is added (the loads
            // overlap); the sum still runs over the splits in order
#pragma unroll 1
            for (int p0 = 1; p0 < nsplit; p0 += BATCH) {
                float q[BATCH][EPL];
#pragma unroll
                for (int u = 0; u < BATCH; ++u) {
                    if (p0 + u < nsplit) {
                        load_run<EPL, FULL>(partials + (p0 + u) * plane + row, vec, n, q[u]);
                    } else {
#pragma unroll
                        for (int i = 0; i < EPL; ++i) q[u][i] = 0.f;
                    }
                }
#pragma unroll
                for (int u = 0; u < BATCH; ++u)
                    if (p0 + u < nsplit) {
#pragma unroll
                        for (int i = 0; i < EPL; ++i) lg[i] += q[u][i];
                    }
            }
#pragma unroll
            for (int i = 0; i < EPL; ++i) {
                lg[i] *= scale;
                if (i < n) logits[row + i] = lg[i];
            }
        }
    }
    uint32_t key[EPL];
    uint32_t live = 0;   // bit i: expert EPL*lane + i still a candidate
#pragma unroll
    for (int i = 0; i < EPL; ++i) {
        key[i] = 0u;
        if (valid && i < n) {
            key[i] = ordered_key(sigmoid_rn(lg[i]) + bias[e0 + i]);
            live |= 1u << i;
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
    // full lanes of a valid token: every expert of the lane is a candidate
    if constexpr (FULL) live = (1u << EPL) - 1u;

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
        // The k-th largest key: the largest v with at least k candidates
        // whose key is >= v, found bit by bit from the top (each step counts
        // with one ballot per register slot; the count and the bound stay
        // scalar). Every key shares the bits above the highest bit where the
        // smallest and the largest key differ, so the search starts below.
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
#pragma unroll 1
        for (int b = top; b >= 0; --b) {
            const uint32_t cand = thr | (1u << b);
            int cnt = 0;
#pragma unroll
            for (int i = 0; i < EPL; ++i) cnt += __popcll(__ballot(((live >> i) & 1u) && key[i] >= cand));
            if (cnt >= k) thr = cand;
        }
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
}

// Any E: each wave stages its token's keys in its own LDS region (dynamic
// LDS: kSelectWaves * E * 4 bytes). A lane only touches the entries of its
// own experts, so no barrier is needed. The picks' logits are read back from
// the token's logit row at the end (the caller's logits, or the row this
// wave has just written), which keeps the LDS per block at one key per
// expert and lets four blocks share a CU at 2560 experts.
__global__ __launch_bounds__(kSelectBlock) void select_lds_kernel(
    const float* __restrict__ partials, int nsplit, float scale, int logits_in,
    const float* __restrict__ bias, const uint8_t* __restrict__ token_mask, int T, int E, int k,
    float* __restrict__ logits, int32_t* __restrict__ topk_ids, float* __restrict__ topk_w) {
    extern __shared__ uint32_t sel_lds[];
    const int lane = __lane_id();
    const int wave = threadIdx.x / kWave;
    const int t = blockIdx.x * kSelectWaves + wave;
    if (t >= T) return;
    uint32_t* keys = sel_lds + static_cast<size_t>(wave) * E;
    const size_t plane = static_cast<size_t>(T) * E;
    const bool valid = token_mask[t] != 0;
    // the lane's experts e = lane + 64 i, kLdsBatch at a time: their logits
    // (or split partials, split by split) are all loaded before any is used,
    // so the loads overlap; each logit still sums its splits in order
#pragma unroll 1
    for (int e0 = lane; e0 < E; e0 += kLdsBatch * kWave) {
        float l[kLdsBatch];
#pragma unroll
        for (int u = 0; u < kLdsBatch; ++u) {
            const int e = e0 + u * kWave;
            const size_t idx = static_cast<size_t>(t) * E + e;
            l[u] = e < E ? (logits_in ? logits[idx] : partials[idx]) : 0.f;
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
            for (int u = 0; u < kLdsBatch; ++u) {
                const int e = e0 + u * kWave;
                l[u] *= scale;
                if (e < E) logits[static_cast<size_t>(t) * E + e] = l[u];
            }
        }
#pragma unroll
        for (int u = 0; u < kLdsBatch; ++u) {
            const int e = e0 + u * kWave;
            if (e < E) keys[e] = valid ? ordered_key(sigmoid_rn(l[u]) + bias[e]) : 0u;
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
    const int nloc = lane < E ? (E - lane + kWave - 1) / kWave : 0;   // <= 64
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
    // lane j < k reads pick j's logit from the row (written above by the
    // lane that owns the expert, so the wave's stores are made visible first)
    __threadfence_block();
    const float my_l = lane < k ? logits[static_cast<size_t>(t) * E + my_id] : 0.f;
    write_picks(lane, k, my_id, my_l, ids, w);
}

template <int EPL, int BATCH>
int launch_select_reg2(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
                       const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
                       void* stream) {
    const dim3 grid(ceil_div(T, kSelectWaves));
#define MOE_SELECT(THR, FULL)                                                                                 \
    return launch(select_reg_kernel<EPL, BATCH, THR, FULL>, grid, dim3(kSelectBlock), 0, stream, partials, nsplit, \
                  scale, logits_in, bias, mask, T, E, k, logits, ids, w)
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
                      void* stream) {
    if (nsplit > 2 * kSplitBatch)
        return launch_select_reg2<EPL, 4 * kSplitBatch>(partials, nsplit, scale, logits_in, bias, mask, T, E, k,
                                                        logits, ids, w, stream);
    return launch_select_reg2<EPL, kSplitBatch>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits,
                                                ids, w, stream);
}

}  // namespace

int run_select(const float* partials, int nsplit, float scale, int logits_in, const float* bias,
               const uint8_t* mask, int T, int E, int k, float* logits, int32_t* ids, float* w,
               void* stream) {
    const int epl = ceil_div(E, kWave);
    if (epl <= 1) return launch_select_reg<1>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, stream);
    if (epl <= 2) return launch_select_reg<2>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, stream);
    if (epl <= 4) return launch_select_reg<4>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, stream);
    if (epl <= 8) return launch_select_reg<8>(partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w, stream);
    const size_t lds = static_cast<size_t>(kSelectWaves) * E * sizeof(uint32_t);
    return launch(select_lds_kernel, dim3(ceil_div(T, kSelectWaves)), dim3(kSelectBlock), lds, stream,
                  partials, nsplit, scale, logits_in, bias, mask, T, E, k, logits, ids, w);
}

}  // namespace moe
