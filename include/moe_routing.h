/*
 * moe_routing.h — C ABI of the MoE routing-and-combine hot path on MI355X
 * (gfx950).
 *
 * The four calls, in pipeline order:
 *
 *   moe_route             router projection, sigmoid + bias selection, sorted
 *                         top-k with lowest-id ties, renormalised weights,
 *                         per-token validity mask
 *   moe_dispatch          expert histogram, exclusive prefix scan, stable
 *                         permutation of the routed slots by expert
 *                         (moe_dispatch_noalloc: the same without a workspace,
 *                         for callers that cannot allocate)
 *   moe_route_dispatch    moe_route followed by moe_dispatch in one call, the
 *                         selection counting the dispatch's tile histograms
 *                         (moe_route_dispatch_quant: and moe_norm_quant_nvfp4
 *                         of the expert input, the dispatch's last step and
 *                         the norm + quant sharing one launch)
 *   moe_norm_quant_nvfp4  RMSNorm of the expert input with one BF16 rounding,
 *                         fused with NVFP4 quantisation (E2M1 codes, E4M3
 *                         block-16 scales, static global scale); the
 *                         _rank_block variant reads the input in the
 *                         [tp*T, H/tp] layout a column all-gather leaves
 *   moe_combine           per-row RMSNorm of each selected expert output,
 *                         routing-weight scaling and top-k sum; invalid slots
 *                         are never read
 *
 * and, beside the path, the expert FC1 the dispatch feeds:
 *
 *   moe_expert_fc1_nvfp4  gather grouped GEMM of the NVFP4 input with NVFP4
 *                         per-expert weights, Relu2, NVFP4 output
 *   moe_expert_fc1_swiglu_nvfp4
 *                         the same GEMM over gate and up weight rows, SwiGLU,
 *                         NVFP4 output
 *
 * Conventions shared by every call:
 *   - Every array argument is a DEVICE pointer (memory the caller allocated on
 *     the current HIP device), row-major, contiguous and 16-byte aligned
 *     (MOE_ERR_ALIGN otherwise). The caller owns all
 *     memory; the library never allocates, frees or synchronises, and keeps no
 *     state between calls (moe_dispatch_noalloc's static device scratch, the
 *     one exception, is described with it).
 *   - `stream` is the caller's hipStream_t (NULL = the null stream). Work is
 *     enqueued on it; the call returns without waiting.
 *   - The return value is MOE_OK (0) or a negative MOE_ERR_* status. Every
 *     argument check runs before any work is enqueued, so a failing call
 *     leaves every output untouched. MOE_ERR_HIP reports a failed launch.
 *   - BF16 values are passed as their uint16_t bit patterns.
 *   - T == 0 (no tokens) is valid and enqueues nothing.
 *   - Outputs are fully written; nothing needs clearing beforehand.
 *   - Shapes are run-time arguments; nothing is compiled per token count.
 */
#ifndef MOE_ROUTING_H
#define MOE_ROUTING_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

enum moe_status {
    MOE_OK = 0,
    MOE_ERR_NULL_ARG = -1,   /* a required pointer is NULL */
    MOE_ERR_BAD_SHAPE = -2,  /* a size is out of the supported range */
    MOE_ERR_BAD_DTYPE = -3,  /* unknown dtype code */
    MOE_ERR_WORKSPACE = -4,  /* workspace missing or smaller than required */
    MOE_ERR_BAD_ARG = -5,    /* a scalar argument is out of range (eps, scale) */
    MOE_ERR_HIP = -6,        /* the HIP runtime rejected a launch */
    MOE_ERR_ALIGN = -7       /* an array pointer is not 16-byte aligned */
};

enum moe_dtype {
    MOE_DTYPE_F32 = 0,
    MOE_DTYPE_BF16 = 1
};

/* Supported ranges (checked by every call). */
#define MOE_MAX_EXPERTS 4096
#define MOE_MAX_TOPK 32
#define MOE_MAX_HIDDEN 16384

/* Text for a status code (static storage; never NULL). */
const char* moe_status_string(int status);

/*
 * moe_route — router projection and routing.
 *
 * Defined by TensorRT-LLM PR #21356 ("Add the Muse Spark Open decoder fast
 * paths"), description, Triton kernels "Router projection" (FP32 weights and
 * accumulation, input cast and scale folded in) and "Routing" (sigmoid, bias,
 * top-k, renormalised weights; picks sorted, exact ties to the lowest id); by
 * TensorRT-LLM PR #21042 ("Add the Muse Spark Open model"), "MoE" (the router
 * runs in FP32); and by lmdeploy PR #4835 (MoE gate v2: a required per-token
 * validity mask, invalid tokens produce no routing entries; the aux-loss-free
 * gate uses the bias for selection only).
 *
 * For every token t and expert e:
 *   logits[t,e] = scale * sum_i hidden[t,i] * W[e,i]      FP32 accumulation
 *   s[t,e]      = sigmoid(logits[t,e])                    correctly rounded FP32
 *   key[t,e]    = s[t,e] + bias[e]                        FP32
 * topk_ids[t,:] are the k experts with the largest keys, ordered by key
 * (largest first), equal keys by ascending expert id.
 * topk_w[t,j]  = s[t,id_j] / (s[t,id_0] + ... + s[t,id_{k-1}])   (FP32 sum in
 * pick order, one FP32 division).
 * token_mask[t] == 0: topk_ids[t,:] = -1 and topk_w[t,:] = 0.0; such a token's
 * input is never inspected (it may hold NaN).
 *
 * Arguments:
 *   hidden        [T,H] in hidden_dtype (MOE_DTYPE_BF16 bits or MOE_DTYPE_F32),
 *                 or NULL for logits-in mode: `logits` is then an INPUT [T,E]
 *                 and the projection is skipped.
 *   W             [E,H] FP32 router weight (nn.Linear orientation). Unused in
 *                 logits-in mode (may be NULL).
 *   bias          [E] FP32 selection bias (required).
 *   token_mask    [T] u8, nonzero = valid (required).
 *   scale         finite scale applied to the dot products (1.0 for none).
 *   T >= 0, 1 <= H <= MOE_MAX_HIDDEN with H % 16 == 0,
 *   1 <= E <= MOE_MAX_EXPERTS, 1 <= k <= min(E, MOE_MAX_TOPK).
 *   logits        [T,E] FP32: output (projection mode) or input (logits-in).
 *                 In projection mode the rows of invalid tokens hold whatever
 *                 their (possibly NaN) input gives.
 *   topk_ids      [T,k] int32 output; topk_w [T,k] FP32 output.
 *   workspace     device scratch of at least moe_route_workspace_bytes(...)
 *                 bytes (may be NULL when that is 0); 256-byte aligned.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_DTYPE, BAD_ARG (non-finite scale),
 * WORKSPACE, HIP.
 */
size_t moe_route_workspace_bytes(int T, int H, int E, int k, int hidden_dtype, int logits_in);

int moe_route(const void* hidden, int hidden_dtype, const float* W, const float* bias,
              const uint8_t* token_mask, float scale, int T, int H, int E, int k,
              float* logits, int32_t* topk_ids, float* topk_w,
              void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_dispatch — histogram, scan and permutation of the routed slots.
 *
 * Defined by lmdeploy PR #4835 ("Intern-S2-Mobius meta-MoE support, MoE gate
 * v2, CP attention fixes"): the gate's shared-memory expert histogram and
 * hierarchical multi-block scan over tiles, the required validity mask
 * (invalid tokens get no entry), and the slot-to-position map cleared to -1.
 *
 * Slot f = t*k + j is valid when 0 <= topk_ids[t,j] < E.
 *   counts[e]     number of valid slots routed to expert e          [E]
 *   offsets[e]    exclusive prefix sum of counts; offsets[E] = valid slots
 *                                                                    [E+1]
 *   perm[p]       flat slot at position p: slots grouped by ascending expert,
 *                 ascending flat index within an expert (stable); -1 for
 *                 p >= offsets[E]                                    [T*k]
 *   dest[f]       position of slot f, or -1 if slot f is not valid   [T*k]
 * All outputs int32 and fully written. T >= 0, 1 <= k <= MOE_MAX_TOPK,
 * 1 <= E <= MOE_MAX_EXPERTS, T*k < 2^31. The result is deterministic.
 * workspace: at least moe_dispatch_workspace_bytes(T, k, E) bytes.
 * Errors: NULL_ARG, BAD_SHAPE, WORKSPACE, HIP.
 */
size_t moe_dispatch_workspace_bytes(int T, int k, int E);

int moe_dispatch(const int32_t* topk_ids, int T, int k, int E,
                 int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* dest,
                 void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_dispatch — moe_route, then moe_dispatch of its topk_ids, in one
 * call.
 *
 * Defined by the two calls above: TensorRT-LLM PR #21356, "Router
 * projection" and "Routing", for the route; lmdeploy PR #4835, MoE gate v2
 * notes, for the dispatch, whose gate fuses the expert histogram into the
 * pass that produces the ids. Here the selection adds each valid pick into
 * the histogram of its tile of slots as it writes it (integer atomics, so
 * the counts do not depend on arrival order), and the separate histogram
 * pass of moe_dispatch is skipped. The projection clears those histograms
 * first (in logits-in mode a small kernel does).
 *
 * Arguments: those of moe_route, then the four outputs of moe_dispatch
 * (counts [E], offsets [E+1], perm [T*k], dest [T*k]); same meaning, layout,
 * ranges and checks as in the two calls. Every output is bit-identical to
 * moe_route followed by moe_dispatch on the same inputs.
 *   workspace   at least moe_route_dispatch_workspace_bytes(T, H, E, k,
 *               hidden_dtype, logits_in) bytes (may be NULL when that is 0):
 *               moe_route's workspace, then the tile histograms.
 * Errors: those of either call.
 */
size_t moe_route_dispatch_workspace_bytes(int T, int H, int E, int k, int hidden_dtype, int logits_in);

int moe_route_dispatch(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                       const uint8_t* token_mask, float scale, int T, int H, int E, int k,
                       float* logits, int32_t* topk_ids, float* topk_w,
                       int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* dest,
                       void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_route_dispatch_quant — moe_route_dispatch, then moe_norm_quant_nvfp4 of
 * the expert input, in one call: what the experts need of a batch.
 *
 * TensorRT-LLM PR #21356, "Where they plug in": the expert input's norm and
 * quantisation run beside the routing (on an auxiliary stream there). Here
 * the dispatch's place step and the norm + quant share one launch, blocks of
 * each side by side, when x's rows fill a wave or whole 256-thread blocks
 * (Hq / 16 = 64, 256, 512, 768 or 1024) or every slot lies in one dispatch
 * tile; otherwise they run one after the other. Same outputs either way:
 * every output is bit-identical to moe_route_dispatch followed by
 * moe_norm_quant_nvfp4.
 *
 * Arguments: those of moe_route_dispatch, then those of moe_norm_quant_nvfp4
 * for the expert input x [T,Hq] BF16 (the same T as hidden; its own width
 * Hq, since the experts may read a narrower stream than the router, e.g. a
 * pooled one; contiguous rows): norm_w [Hq] FP32, gain_center, eps,
 * global_scale (one FP32 on the device), packed [T,Hq/2], scales [T,Hq/16].
 * workspace: at least moe_route_dispatch_workspace_bytes(T, H, E, k,
 * hidden_dtype, logits_in). Errors: those of either call (Hq checked as
 * moe_norm_quant_nvfp4 checks H).
 */
int moe_route_dispatch_quant(const void* hidden, int hidden_dtype, const float* W, const float* bias,
                             const uint8_t* token_mask, float scale, int T, int H, int E, int k,
                             float* logits, int32_t* topk_ids, float* topk_w,
                             int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* dest,
                             const uint16_t* x, int Hq, const float* norm_w, float gain_center, float eps,
                             const float* global_scale, uint8_t* packed, uint8_t* scales,
                             void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_dispatch_noalloc — moe_dispatch without a workspace argument, for
 * callers that cannot allocate device memory (code under HIP graph capture,
 * tight serving loops, harnesses that forbid hipMalloc).
 *
 * Same operation, arguments (minus workspace), outputs, checks and kernels as
 * moe_dispatch. The per-tile histogram scratch is a static device array of
 * the library, 4 MiB (256 tiles x MOE_MAX_EXPERTS int32; every shape
 * moe_dispatch accepts fits), one copy per GPU the library runs on, held
 * until the process ends; its device address is looked up once per device
 * (hipGetSymbolAddress) on the first call there. Nothing is allocated or
 * freed. Every call on one GPU shares that GPU's array, which keeps the last
 * call's contents (each call writes every entry it reads, so nothing needs
 * clearing): calls that may overlap on one GPU -- on different streams, or
 * from different host threads without ordering -- race and must not be
 * issued. A shape needing more scratch than the array would be rejected
 * with WORKSPACE.
 * Errors: NULL_ARG, BAD_SHAPE, ALIGN, WORKSPACE, HIP.
 */
int moe_dispatch_noalloc(const int32_t* topk_ids, int T, int k, int E,
                         int32_t* counts, int32_t* offsets, int32_t* perm, int32_t* dest,
                         void* stream);

/*
 * moe_norm_quant_nvfp4 — RMSNorm + NVFP4 quantisation of the expert input.
 *
 * Defined by the vLLM API docs of vllm.models.muse_spark.nvidia.ops.
 * prepare_trtllm_nvfp4 (`norm_quant_trtllm_nvfp4` and the block quantizer
 * `_quantize_nvfp4_global_scale`) and TensorRT-LLM PR #21356, "Numerics" (the
 * gain centre is added to the weight in FP32, the norm rounds only its
 * result to BF16).
 *
 * Per row t:  g_i = gain_center + norm_w[i]                  FP32
 *             y_i = bf16( x_i * g_i / sqrt(mean_i(x_i^2) + eps) )
 * Per block of 16 consecutive y (all FP32 steps, IEEE-rounded reciprocals):
 *             sf   = e4m3_satfinite( gs * (amax|y| * (1/6)) )
 *             out  = sf != 0 ? 1 / (sf * (1/gs)) : 0
 *             code = e2m1_rne_saturating(y * out), bit 3 set when y*out < 0
 * packed[t, i/2] holds code(2m) in its low nibble and code(2m+1) in its high
 * nibble; scales[t, b] is the E4M3 byte of block b (linear layout).
 *
 *   x            [T,H] BF16 bits.   norm_w [H] FP32.
 *   gain_center  finite FP32.       eps >= 0, finite (0 allowed).
 *   global_scale device pointer to ONE FP32 value gs > 0 (static scale).
 *   T >= 0, 16 <= H <= MOE_MAX_HIDDEN, H % 16 == 0.
 *   packed [T, H/2] u8 output; scales [T, H/16] u8 output.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_ARG, HIP.
 */
int moe_norm_quant_nvfp4(const uint16_t* x, const float* norm_w, float gain_center, float eps,
                         const float* global_scale, int T, int H,
                         uint8_t* packed, uint8_t* scales, void* stream);

/*
 * moe_norm_quant_nvfp4_rank_block — the same operation on input in the
 * rank-block layout.
 *
 * Defined by the vLLM API docs of vllm.models.muse_spark.nvidia.ops.
 * prepare_trtllm_nvfp4 (module description and `norm_quant_trtllm_nvfp4`):
 * the pooled input is either [M, H] or the [tp * M, H / tp] result of a
 * dim-0 all-gather of column shards, i.e. tp blocks of [M, H / tp], block r
 * holding columns [r * shard, (r + 1) * shard) of every row.
 *
 *   x      [H/shard * T, shard] BF16 bits: element (t, i) of the logical
 *          [T,H] input is x[(i / shard) * T + t, i % shard].
 *   shard  columns per rank block: 16 <= shard <= H, shard % 16 == 0 (an
 *          NVFP4 block never straddles two shards) and H % shard == 0.
 *          shard == H is the contiguous layout and gives moe_norm_quant_nvfp4.
 *   Every other argument, the outputs (packed and scales in the logical
 *   [T, ...] layout) and the errors are those of moe_norm_quant_nvfp4;
 *   a shard outside these rules is BAD_SHAPE.
 */
int moe_norm_quant_nvfp4_rank_block(const uint16_t* x, int shard, const float* norm_w,
                                    float gain_center, float eps, const float* global_scale,
                                    int T, int H, uint8_t* packed, uint8_t* scales, void* stream);

/*
 * moe_combine — post-expert RMSNorm, weighting and top-k sum.
 *
 * Defined by TensorRT-LLM PR #21356, description, Triton kernel "Post-expert
 * norm and combine" (weight-first RMSNorm of each selected expert row, the
 * routing weights and the top-k sum per token; a row behind an invalid slot —
 * negative or past the end of the expert output — is never read) and
 * "Routing" (the pick order fixes the summation order); TensorRT-LLM PR
 * #21042, "MoE" (post-expert RMSNorm of each expert output before the
 * weighted top-k sum).
 *
 * For token t, over j = 0..k-1 in order, with r = slots[t,j]:
 *   skip unless 0 <= r < R (row r of expert_out is then never read)
 *   z   = bf16( expert_out[r,:] * g / sqrt(mean(expert_out[r,:]^2) + eps) ),
 *         g = gain_center + norm_w (FP32)
 *   acc += topk_w[t,j] * z                  (FP32)
 * out[t,:] = bf16(acc); a token with no valid slot gets +0.0.
 *
 *   expert_out [R,H] BF16 bits (R >= 0; may be NULL only if R == 0).
 *   slots      [T,k] int32 (typically moe_dispatch's dest viewed as [T,k]).
 *   topk_w     [T,k] FP32.   norm_w [H] FP32.
 *   gain_center finite, eps >= 0 finite.
 *   T >= 0, 1 <= k <= MOE_MAX_TOPK, 8 <= H <= MOE_MAX_HIDDEN, H % 8 == 0.
 *   out [T,H] BF16 bits output.
 * Errors: NULL_ARG, BAD_SHAPE, BAD_ARG, HIP.
 */
int moe_combine(const uint16_t* expert_out, int R, const int32_t* slots, const float* topk_w,
                const float* norm_w, float gain_center, float eps, int T, int H, int k,
                uint16_t* out, void* stream);

/*
 * moe_expert_fc1_nvfp4 — the expert FC1 on the dispatched NVFP4 input: a
 * gather grouped GEMM per expert, Relu2, NVFP4 output.
 *
 * Defined by TensorRT-LLM PR #21842 ("CuTe DSL act-fusion GEMMs: key the
 * early accumulator release on the loop index"), description: the NVFP4 MoE
 * FC1 is a block-scaled gather grouped GEMM with a fused activation (Relu2 on
 * its K 1024, N 2688, 512-expert, top-22 workload) whose outputs are FP4
 * values and their scale factors; the NVFP4 format and block quantiser are
 * those of moe_norm_quant_nvfp4; the grouping is moe_dispatch's.
 *
 * For grouped position p < offsets[E], expert e with offsets[e] <= p <
 * offsets[e+1], token t = perm[p] / k, and n < N:
 *   v[p,n] = sum_i xv(t,i) * wv(e,n,i),  xv = code * scale / x_gs,
 *                                         wv = code * scale / w_gs[e]
 *   y[p,n] = max(v, 0)^2                  (FP32 accumulation)
 * y is quantised per 16 consecutive n with the static scale y_gs exactly as
 * moe_norm_quant_nvfp4 quantises its normalised rows. Positions p >=
 * offsets[E] get zero codes and zero scales.
 *
 *   x_packed [T, K/2] u8, x_scales [T, K/16] u8 (E4M3): the NVFP4 input of
 *            each token (moe_norm_quant_nvfp4's output); x_gs -> one FP32.
 *   perm [T*k], offsets [E+1]: moe_dispatch's outputs for the same T, k, E.
 *   w_packed [E, N, K/2] u8, w_scales [E, N, K/16] u8: per-expert weights
 *            (output features x input features, NVFP4 along K);
 *            w_gs [E] FP32 (device).
 *   y_gs -> one FP32 (device): static output global scale.
 *   y_packed [T*k, N/2] u8, y_scales [T*k, N/16] u8: outputs, rows in
 *            grouped (perm) order.
 *   T >= 0, 1 <= k <= MOE_MAX_TOPK, 1 <= E <= MOE_MAX_EXPERTS,
 *   64 <= K <= MOE_MAX_HIDDEN with K % 64 == 0, N >= 128 with N % 128 == 0.
 *   x_packed, w_packed, y_packed, y_scales, workspace 16-byte aligned;
 *   x_scales, w_scales 4-byte aligned.
 *   workspace: at least moe_expert_fc1_workspace_bytes(T, k, E) bytes
 *            (per-expert tile starts and one 16-byte record per row tile of
 *            256 grouped rows; 0 means T, k or E is out of range).
 * A perm entry outside [0, T*k) reads no input (its row is computed from
 * zeros); NaN scale bytes (0x7F, 0xFF) in the inputs are not supported.
 * Errors: NULL_ARG, BAD_SHAPE, ALIGN, WORKSPACE, HIP.
 */
size_t moe_expert_fc1_workspace_bytes(int T, int k, int E);

int moe_expert_fc1_nvfp4(const uint8_t* x_packed, const uint8_t* x_scales, const float* x_gs,
                         const int32_t* perm, const int32_t* offsets, int T, int k,
                         const uint8_t* w_packed, const uint8_t* w_scales, const float* w_gs,
                         const float* y_gs, int K, int N, int E,
                         uint8_t* y_packed, uint8_t* y_scales,
                         void* workspace, size_t workspace_bytes, void* stream);

/*
 * moe_expert_fc1_swiglu_nvfp4 — the expert FC1 with SwiGLU instead of Relu2.
 *
 * Defined by the same TensorRT-LLM PR #21842 description, which names SwiGLU
 * as the gather grouped GEMM's other fused activation without giving its
 * weight layout. The layout taken here: each expert's weights hold 2N rows,
 * the gate projection's N rows first, then the up projection's N rows.
 *
 * For grouped position p < offsets[E] (expert e, token t as in
 * moe_expert_fc1_nvfp4) and output column n < N:
 *   g = sum_i xv(t,i) * wv(e,n,i),   u = sum_i xv(t,i) * wv(e,N+n,i)
 *   y[p,n] = silu(g) * u,  silu(g) = g / (1 + exp(-g))   (FP32 evaluation)
 * y is quantised per 16 consecutive n with the static scale y_gs exactly as
 * moe_norm_quant_nvfp4 quantises its rows; positions p >= offsets[E] get zero
 * codes and zero scales.
 *
 *   w_packed [E, 2N, K/2] u8, w_scales [E, 2N, K/16] u8: gate rows 0..N-1,
 *            up rows N..2N-1 of each expert; w_gs [E] FP32 (device).
 *   y_packed [T*k, N/2] u8, y_scales [T*k, N/16] u8: outputs, rows in
 *            grouped (perm) order.
 *   Every other argument, the ranges of T, k, E and K, the alignments and
 *   the workspace are those of moe_expert_fc1_nvfp4 (the same
 *   moe_expert_fc1_workspace_bytes); N >= 64 with N % 64 == 0.
 * Errors: NULL_ARG, BAD_SHAPE, ALIGN, WORKSPACE, HIP.
 */
int moe_expert_fc1_swiglu_nvfp4(const uint8_t* x_packed, const uint8_t* x_scales, const float* x_gs,
                                const int32_t* perm, const int32_t* offsets, int T, int k,
                                const uint8_t* w_packed, const uint8_t* w_scales, const float* w_gs,
                                const float* y_gs, int K, int N, int E,
                                uint8_t* y_packed, uint8_t* y_scales,
                                void* workspace, size_t workspace_bytes, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* MOE_ROUTING_H */
