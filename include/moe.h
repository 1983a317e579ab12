/*
 * moe.h -- C ABI of the MI355X (gfx950) MoE layer forward pass.
 *
 * One MoE layer, as described on the pages this library follows:
 *   [NOTES] "MoE notes: what one token goes through in an MoE layer"
 *           (www.cf-1.com/news/5905749)
 *   [ENG]   "MoE 大模型推理工程深度实践：专家路由、负载均衡与分布式部署"
 *           (ybb.press/quantum-computing/18594)
 *   [SERVE] MoE inference serving essay (www.dpshk.com/news/3211971)
 *
 *   route    : logits = x W_r; l' = logits + bias; softmax over all E experts;
 *              the K largest (lower expert index first on ties); the K scores
 *              renormalised to sum to one.       [NOTES] §1.2, §2 steps 1-3
 *   dispatch : (token, slot) assignments grouped per expert by histogram,
 *              prefix sum and a stable scatter, optional capacity cut in
 *              token order; token rows gathered into the grouped buffer.
 *                                                 [NOTES] §2.1, §3.1
 *   expert   : per expert e, SwiGLU FFN h = W2_e (SiLU(W1_e a) * (W3_e a)) on
 *              that expert's rows, as a grouped GEMM.   [NOTES] §2 step 3
 *   combine  : y[t] = sum_k w[t,k] h[t,k] back in token order.
 *                                                 [NOTES] §2 step 4, §2.3
 *   aux/bias : aux = E sum_e f_e P_e ([NOTES] §1.2); per-expert bias +-alpha
 *              toward the average load ([ENG] §1.2).
 *
 * Conventions (all entry points):
 *  - Every tensor pointer is a DEVICE pointer to caller-owned, row-major
 *    memory, 16-byte aligned.  The library never allocates, frees or keeps
 *    per-call state; scratch memory comes in through `ws` / `ws_bytes`.
 *  - `stream` is a hipStream_t (NULL = the default stream).  Calls only
 *    enqueue work on it and return; they never synchronise.  Results are valid
 *    once the caller synchronises the stream.
 *  - Argument checks run on the host before any launch and return a status
 *    (no work is enqueued when the status is not MOE_OK).  A failed launch
 *    returns MOE_ERR_HIP.  Faults inside kernels surface at the caller's next
 *    synchronisation, as usual with HIP.
 *  - Element types: x, weights, x_perm, act, h and y use `dtype`
 *    (fp32 or bf16); logits, probabilities, routing weights and biases are
 *    fp32; ids, counts, offsets and row maps are int32.
 *  - Non-finite inputs are outside the contract.
 *  - Calls on distinct workspaces are independent and re-entrant.  The one
 *    piece of process-wide state is the tracing hook moe_set_kernel_timer:
 *    while it is armed, launches from every thread record into the same
 *    event list (under a lock), so arm it only around single-threaded
 *    measurements.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    MOE_OK = 0,
    MOE_ERR_INVALID_ARG = 1,  /* null pointer, bad size or relation between sizes */
    MOE_ERR_UNSUPPORTED = 2,  /* valid request outside what this build supports */
    MOE_ERR_ALIGNMENT = 3,    /* a pointer is not 16-byte aligned */
    MOE_ERR_WORKSPACE = 4,    /* ws is NULL or ws_bytes is below the required size */
    MOE_ERR_HIP = 5           /* a HIP runtime call or launch failed */
} moe_status;

typedef enum { MOE_DTYPE_F32 = 0, MOE_DTYPE_BF16 = 1 } moe_dtype;

enum { MOE_FLAG_BIAS_SELECT_ONLY = 1u, MOE_FLAG_COMBINE_MEAN = 2u };

/* Shape and options of one layer call.
 *   T         tokens (rows of x), T >= 1, T * top_k < 2^30
 *   d_model   d, multiple of 8, <= 65536
 *   n_experts E, 1 <= E <= 1024
 *   top_k     K, 1 <= K <= min(E, 32)
 *   d_ff      F, multiple of 8, <= 65536
 *   dtype     moe_dtype of activations and expert / router weights; fp32
 *             (the small-layer path) also needs T*K*max(d, F) <= 2^31 and
 *             T*E <= 2^31
 *   capacity  < 0: unlimited; >= 0: at most `capacity` rows kept per expert,
 *             in flat assignment order t*K + k ([NOTES] §3.1: a capacity
 *             factor cf gives capacity = floor(cf * T * K / E), computed by the
 *             caller)
 *   flags     0, or an OR of
 *             MOE_FLAG_BIAS_SELECT_ONLY: the logit bias steers which experts
 *               are chosen, while the probabilities and the weights come from
 *               the softmax of the unbiased scores ([ENG] §1.2 read as a
 *               routing-only bias; without the flag the bias enters both);
 *             MOE_FLAG_COMBINE_MEAN: the K outputs are averaged without
 *               weights, every routing weight is 1/K ([NOTES] §2.3). */
typedef struct {
    int32_t T;
    int32_t d_model;
    int32_t n_experts;
    int32_t top_k;
    int32_t d_ff;
    int32_t dtype;
    int32_t capacity;
    uint32_t flags;
} moe_problem;

/* Optional device outputs of moe_forward; any field may be NULL, in which
 * case the value lives only in the workspace (z_loss and aux_topk are then
 * not computed).  Shapes as in the step calls.  Pointers are 16-byte aligned,
 * except the two scalars (4-byte aligned). */
typedef struct {
    float* logits;        /* [T, E]  router scores x W_r (before the bias) */
    float* probs;         /* [T, E]  softmax over all experts of logits + bias */
    float* prob_sum;      /* [E]     sum over tokens of probs (for the aux loss) */
    int32_t* topk_ids;    /* [T, K] */
    float* topk_w;        /* [T, K] */
    int32_t* counts;      /* [E] */
    int32_t* kept;        /* [E] */
    int32_t* offsets;     /* [E + 1] */
    int32_t* assign_row;  /* [T * K] */
    int32_t* row_assign;  /* [T * K] */
    /* Router regularisers of [NOTES] §3.2, gathered by the routing kernel from
     * its own max and sum of exponentials (one fp32 each, as
     * moe_router_losses defines them): */
    float* z_loss;        /* (1/T) sum_t (log sum_e exp(logits[t,e]))^2 */
    float* aux_topk;      /* E sum_e f_e P'_e over the chosen experts */
} moe_debug_out;

/* Human-readable name of a status. */
const char* moe_status_string(moe_status s);

/* Library version string. */
const char* moe_version(void);

/* Workspace bytes needed by moe_route (when it computes bf16 scores from x,
 * or when prob_sum is requested), moe_dispatch, moe_expert_ffn and
 * moe_forward for problem `p`. */
moe_status moe_route_workspace_size(const moe_problem* p, size_t* bytes);
moe_status moe_dispatch_workspace_size(const moe_problem* p, size_t* bytes);
moe_status moe_expert_ffn_workspace_size(const moe_problem* p, size_t* bytes);
moe_status moe_workspace_size(const moe_problem* p, size_t* bytes);

/* Router: [NOTES] §1.2 (router_forward: scores = softmax(x W_r)), §2 steps
 * 1-3 and §2.1 (softmax over all experts, top-K, renormalise over the K);
 * [ENG] §1 (TopKRouter) and §1.2 (logits = gate(x) + bias).
 *   x          [T, d] dtype, or NULL: then `logits` is an INPUT holding the
 *              router scores and only the routing steps run
 *   w_router   [d, E] dtype (ignored when x is NULL)
 *   logit_bias [E] fp32 or NULL; added to every token's logits before the
 *              softmax and the top-K
 *   logits     [T, E] fp32, out (in when x is NULL): x W_r, fp32 accumulation
 *   probs      [T, E] fp32 or NULL: softmax over all E of logits + bias
 *   prob_sum   [E] fp32 or NULL: sum over tokens of probs (fixed order)
 *   ws         scratch of moe_route_workspace_size bytes; required when x is
 *              given with dtype bf16 or when prob_sum is requested, else may
 *              be NULL
 *   topk_ids   [T, K] int32: experts by (l' descending, index ascending);
 *              -0.0 and +0.0 compare equal
 *   topk_w     [T, K] fp32: p[id_k] / sum_j p[id_j] (1/K with
 *              MOE_FLAG_COMBINE_MEAN) */
moe_status moe_route(const moe_problem* p, const void* x, const void* w_router,
                     const float* logit_bias, float* logits, float* probs,
                     float* prob_sum, int32_t* topk_ids, float* topk_w,
                     void* ws, size_t ws_bytes, void* stream);

/* Dispatch: [NOTES] §2.1 (permute tokens so each expert's tokens are adjacent,
 * via sort + cumulative sum) and §3.1 (capacity cap, overflow dropped).
 *   topk_ids   [T, K] int32 in [0, E) (checked on the device: an id outside
 *              the range is ignored and counted nowhere)
 *   x          [T, d] dtype, or NULL to skip the row gather
 *   counts     [E]    out: routed assignments per expert (before the cap)
 *   kept       [E]    out: min(counts, capacity) (counts when unlimited)
 *   offsets    [E+1]  out: exclusive prefix sum of kept; offsets[E] = S
 *   assign_row [T*K]  out: row of assignment t*K+k in the grouped buffer, or
 *                     -1 when dropped; rows of one expert follow flat order
 *   row_assign [T*K]  out: inverse map, t*K+k for rows < S, -1 beyond
 *   x_perm     [T*K, d] dtype out (may be NULL iff x is NULL): x_perm[row] =
 *                     x[row_assign[row] / K] for rows < S */
moe_status moe_dispatch(const moe_problem* p, const int32_t* topk_ids, const void* x,
                        int32_t* counts, int32_t* kept, int32_t* offsets,
                        int32_t* assign_row, int32_t* row_assign, void* x_perm,
                        void* ws, size_t ws_bytes, void* stream);

/* Grouped expert FFN: [NOTES] §2 step 3 (every expert is an FFN) and §2.3
 * (batched permute, batched GEMM); SwiGLU form h = W2 (SiLU(W1 a) * (W3 a)).
 *   x_perm  [T*K, d] dtype: grouped rows (rows of expert e are
 *           offsets[e] .. offsets[e+1]-1)
 *   offsets [E+1] int32 (device; group sizes are never read on the host)
 *   w1, w3  [E, F, d] dtype;  w2 [E, d, F] dtype
 *   act     [T*K, F] dtype out: SiLU(x_perm W1_e^T) * (x_perm W3_e^T), fp32
 *           accumulation, rounded to dtype
 *   h       [T*K, d] dtype out: act W2_e^T
 * Rows >= offsets[E] of act and h are left untouched. */
moe_status moe_expert_ffn(const moe_problem* p, const void* x_perm, const int32_t* offsets,
                          const void* w1, const void* w3, const void* w2,
                          void* act, void* h, void* ws, size_t ws_bytes, void* stream);

/* Combine: [NOTES] §2 step 4 and §2.3 (weighted sum with a combine mask).
 *   h          [T*K, d] dtype (grouped rows)
 *   assign_row [T*K] int32 (-1 = dropped: contributes nothing)
 *   topk_w     [T, K] fp32
 *   y          [T, d] dtype out: y[t] = sum over k ascending of
 *              topk_w[t,k] * h[assign_row[t*K+k]], fp32 accumulation. */
moe_status moe_combine(const moe_problem* p, const void* h, const int32_t* assign_row,
                       const float* topk_w, void* y, void* stream);

/* Whole layer: route -> dispatch -> expert FFN -> combine on one stream, with
 * every intermediate in `ws` (moe_workspace_size bytes).  The grouped token
 * rows are not materialised here: the expert FFN reads each group's token
 * rows from x through the dispatch's row map ([SERVE] §10.4, a fused MoE
 * kernel avoids the separate permute pass).
 *   x [T,d], w_router [d,E], w1/w3 [E,F,d], w2 [E,d,F] in dtype;
 *   logit_bias [E] fp32 or NULL; y [T,d] dtype out;
 *   dbg: NULL, or device pointers that receive intermediate results. */
moe_status moe_forward(const moe_problem* p, const void* x, const void* w_router,
                       const void* w1, const void* w3, const void* w2,
                       const float* logit_bias, void* y, const moe_debug_out* dbg,
                       void* ws, size_t ws_bytes, void* stream);

/* Allocation-free whole layer, for callers that cannot allocate device
 * memory (code under HIP graph capture, tight serving loops, harnesses that
 * forbid hipMalloc).  The same layer and arguments as moe_forward, except
 * that the workspace is a static device array inside the library, one copy
 * per GPU (MOE_NOALLOC_WS_BYTES bytes, held until the process ends; its
 * address is looked up on the first call on each device).  The call itself
 * allocates nothing: no hipMalloc, no hipFree, no allocating library
 * routine.  Problems whose moe_workspace_size exceeds MOE_NOALLOC_WS_BYTES
 * (decode-sized batches fit: for example 64 tokens of a d = 7168, K = 8,
 * F = 14336 layer need 22 MiB) return MOE_ERR_WORKSPACE before any launch.
 * Every call on one GPU uses that GPU's one array, and nothing in it has to
 * start at zero: calls whose work overlaps on one GPU (concurrent streams,
 * several threads) race on it and must be serialised by the caller. */
#define MOE_NOALLOC_WS_BYTES (32u << 20)
moe_status moe_forward_noalloc(const moe_problem* p, const void* x, const void* w_router,
                               const void* w1, const void* w3, const void* w2,
                               const float* logit_bias, void* y, const moe_debug_out* dbg,
                               void* stream);

/* Chunked forward: [NOTES] §4.3 (chunked MoE for prefill: run the token block
 * in chunks to cap peak memory).  The same layer as moe_forward, run over
 * tokens [t0, t0 + chunk_tokens) one chunk after another on `stream`, with a
 * workspace of moe_forward_chunked_workspace_size bytes (the size for one
 * chunk).  Each token's routing and output are defined as in moe_forward.
 * Capacity must be unlimited (capacity < 0; a per-batch cap does not split
 * into chunks: MOE_ERR_UNSUPPORTED otherwise), and of `dbg` only the
 * per-token fields (logits, probs, topk_ids, topk_w) may be set (the batch
 * sums prob_sum, counts, z_loss and aux_topk are refused with
 * MOE_ERR_INVALID_ARG). */
moe_status moe_forward_chunked_workspace_size(const moe_problem* p, int32_t chunk_tokens,
                                              size_t* bytes);
moe_status moe_forward_chunked(const moe_problem* p, int32_t chunk_tokens, const void* x,
                               const void* w_router, const void* w1, const void* w3,
                               const void* w2, const float* logit_bias, void* y,
                               const moe_debug_out* dbg, void* ws, size_t ws_bytes,
                               void* stream);

/* Aux loss: [NOTES] §1.2, aux = E * sum_e f_e P_e with f_e = counts[e]/(T*K)
 * (counts before any capacity drop) and P_e = prob_sum[e]/T.
 *   counts [E] int32, prob_sum [E] fp32, aux: one fp32 (device). */
moe_status moe_aux_loss(const moe_problem* p, const int32_t* counts, const float* prob_sum,
                        float* aux, void* stream);

/* Bias update: [ENG] §1.2, one step.  For each expert, counts[e]*E > T*K:
 * bias[e] -= alpha; counts[e]*E < T*K: bias[e] += alpha; equal: unchanged
 * (the target is the average T*K/E of [NOTES] §3.1).  fp32 arithmetic.
 *   counts [E] int32, bias [E] fp32 in/out. */
moe_status moe_bias_update(const moe_problem* p, const int32_t* counts, float alpha,
                           float* bias, void* stream);

/* Concatenation combine: [NOTES] §2.3 (the alternative to the weighted sum:
 * concatenate the K expert outputs of a token, then one linear layer).
 *   y[t] = W_cat . concat over k = 0..K-1 of h[assign_row[t,k]]
 * A slot dropped by capacity (assign_row = -1) gives a block of zeros; the
 * routing weights are not used.
 *   h [S,d] grouped expert outputs (as moe_expert_ffn writes them, layer
 *   dtype), assign_row [T,K] int32 (moe_dispatch), W_cat [d, K*d] (layer
 *   dtype, out-features-major like a linear layer's weight), y [T,d] (layer
 *   dtype; bf16 accumulates in fp32 and rounds once).
 *   ws: moe_combine_concat_workspace_size bytes, 16-byte aligned.  Sums run
 *   in a fixed order (run-to-run identical). */
moe_status moe_combine_concat_workspace_size(const moe_problem* p, size_t* bytes);
moe_status moe_combine_concat(const moe_problem* p, const void* h, const int32_t* assign_row,
                              const void* w_cat, void* y, void* ws, size_t ws_bytes, void* stream);

/* Router regularisers: [NOTES] §3.2.
 *   z_loss   = (1/T) sum_t (log sum_e exp(logits[t,e]))^2 over the router
 *              scores as moe_route writes them (before the bias);
 *   aux_topk = E sum_e f_e P'_e, the cheaper aux loss that counts only the
 *              probabilities of the chosen experts: f_e = counts[e] / (T*K),
 *              P'_e = (1/T) sum_t sum_k [topk_ids[t,k] == e] p[t,e] with
 *              p = softmax over all E of logits + logit_bias.
 *   logits [T,E] fp32, logit_bias [E] fp32 or NULL, topk_ids [T,K] int32,
 *   counts [E] int32 (routed, before any capacity cut; may be NULL when
 *   aux_topk is NULL); z_loss, aux_topk: one fp32 each on the device, either
 *   may be NULL.  ws: moe_router_losses_workspace_size bytes.  The sums run
 *   in a fixed order (run-to-run identical). */
moe_status moe_router_losses_workspace_size(const moe_problem* p, size_t* bytes);
moe_status moe_router_losses(const moe_problem* p, const float* logits, const float* logit_bias,
                             const int32_t* topk_ids, const int32_t* counts, float* z_loss,
                             float* aux_topk, void* ws, size_t ws_bytes, void* stream);

/* ---- timing hook (tracing, not part of the layer) -------------------------
 * Kernels of the library, by id, for moe_set_kernel_timer / moe_kernel_name.
 * MOE_KERNEL_FFN times the whole expert FFN (both GEMMs, every launch).
 * MOE_KERNEL_FFN_GATE_UP and MOE_KERNEL_FFN_DOWN time one GEMM step each,
 * with every launch it takes (on large batches, the tiled GEMM, the
 * small-expert launch and the k-split launches of the second GEMM). */
enum {
    MOE_KERNEL_ROUTER = 0,
    MOE_KERNEL_DISPATCH_COUNT = 1,
    MOE_KERNEL_DISPATCH_SCAN = 2,
    MOE_KERNEL_DISPATCH_SCATTER = 3,
    MOE_KERNEL_DISPATCH_GATHER = 4,
    MOE_KERNEL_FFN_GATE_UP = 5,
    MOE_KERNEL_FFN_DOWN = 6,
    MOE_KERNEL_COMBINE = 7,
    MOE_KERNEL_AUX = 8,
    MOE_KERNEL_BIAS_UPDATE = 9,
    MOE_KERNEL_FFN_PLAN = 10,
    MOE_KERNEL_ROUTER_LOSSES = 11,
    MOE_KERNEL_FFN = 12,
    MOE_KERNEL_COUNT = 13
};

/* Name of kernel `kid` ("?" when out of range). */
const char* moe_kernel_name(int kid);

/* While set, each launch of kernel (or GEMM step) `kid`, on whatever stream it runs, is
 * bracketed by hipEventRecord(start_events[i]) / hipEventRecord(stop_events[i])
 * on that stream, for i = 0, 1, ... up to n_events - 1; later launches are not
 * recorded.  The events are hipEvent_t created by the caller.  Passing
 * n_events = 0 clears the hook.  Returns through *recorded (may be NULL) the
 * number of pairs recorded so far when called with n_events < 0 (query only).
 * Process-wide state, guarded by a lock: arming, querying and the recording
 * itself are thread-safe, but launches from several threads while it is
 * armed fill one list in whatever order they run.  While no timer is armed a
 * launch only reads one atomic flag. */
moe_status moe_set_kernel_timer(int kid, void* const* start_events, void* const* stop_events,
                                int n_events, int* recorded);

#ifdef __cplusplus
}
#endif

#endif /* MOE_H */
