/*
 * moe.h -- C ABI of a single-GPU sparse Mixture-of-Experts FFN forward for
 * AMD Instinct MI355X (gfx950).
 *
 * The layer (one forward pass, no training):
 *   1. gate        logits[t][e] = x[t] . w_router[e] (+ router_bias[e])
 *   2. top-k       k experts per token, by the logit (softmax routing) or by
 *                  sigmoid(logit) + sel_bias (sigmoid routing)
 *   3. capacity    optional per-expert limit; (token, expert) pairs beyond it
 *                  are dropped in token order
 *   4. dispatch    kept rows grouped by expert
 *   5. experts     SiLU MLP or GELU MLP with biases, or SwiGLU, plus an
 *                  optional shared expert that every token goes through
 *   6. combine     out[t] = sum_s w[t][s] * y[t][s] (+ shared(x[t]))
 * and, on request, the routing's balance statistics (moe_balance_stats).
 *
 * Sources of each operation are cited at its entry point below: the
 * MoE-router build guide ("Hands-on build guide: pure-Python Mixture-of-
 * Experts router with load-balanced top-k gating"), "Expert Networks > Code
 * Implementation" (Language AI Handbook), "DeepSeek 5.7: MoE from scratch",
 * "Tutorial - MoE SER Expert Routing" and "Implementing Mixed Expert (MoE)
 * Layers in Transformers" (the LLMs-from-scratch MoE guide).
 *
 * Conventions for every entry point
 * ---------------------------------
 * - Every tensor argument is a DEVICE pointer owned by the caller.  The
 *   library never allocates, frees or synchronises; all work is enqueued on
 *   `stream` (a hipStream_t; NULL = the default stream) and is asynchronous.
 *   Results are readable after the caller synchronises the stream.  Since a
 *   call only enqueues kernels (no allocation, copy, fill or synchronisation),
 *   it can be captured into a HIP graph and replayed.
 * - Arguments are validated on the host before anything is enqueued.  On a
 *   non-zero status nothing was enqueued, except MOE_ERR_HIP, which reports
 *   a failed launch.
 * - T = 0 is a successful no-op.  Experts that receive no token are legal.
 * - Row-major layouts.  Weights use the nn.Linear layout [out][in], so every
 *   contraction runs along a contiguous dimension.
 * - "dtype" tensors are float32 or bf16 according to moe_desc.dtype;
 *   routing weights, logits and biases of the router are always float32.
 * - Values in topk_idx passed to moe_dispatch should lie in [0, E) and be
 *   distinct within a token (moe_route guarantees this).  An index outside
 *   [0, E) is dropped (row_of = -1; counted neither as assigned nor kept, so
 *   it shows in n_dropped) and an expert repeated within a token gets one row
 *   per occurrence; moe_check_routing counts the rows that break the
 *   precondition, and a debug build (libmoe_debug.so, moe_debug_checks() = 1)
 *   checks it inside moe_dispatch and returns MOE_ERR_SHAPE.  Logits must be
 *   finite (NaN or infinite logits give unspecified routing).
 * - The library keeps no state between calls; concurrent calls on different
 *   streams need separate workspaces and outputs.
 */
#ifndef MOE_H
#define MOE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

/* ---- status codes -------------------------------------------------------- */
enum {
    MOE_OK = 0,
    MOE_ERR_NULL = 1,        /* a required pointer is NULL                      */
    MOE_ERR_SHAPE = 2,       /* T < 0, k < 1, k > E, d_model or d_ff not a
                                positive multiple of 8, shared width mismatch,
                                x of 2 GiB or more (split such batches into
                                several calls), or one expert matrix or the
                                router of 2 GiB or more                    */
    MOE_ERR_UNSUPPORTED = 3, /* E > 256, unknown dtype / score / expert kind /
                                drop policy, or biases given to SwiGLU
                                experts (which have none)                   */
    MOE_ERR_WORKSPACE = 4,   /* workspace smaller than moe_workspace_size()     */
    MOE_ERR_HIP = 5,         /* a HIP launch failed                             */
    MOE_ERR_TOO_LARGE = 6    /* moe_forward_noalloc: the layer's workspace is
                                larger than moe_scratch_bytes()             */
};

enum { MOE_F32 = 0, MOE_BF16 = 1 }; /* storage dtype */

/* Routing score and weights (see moe_route).  MOE_SCORE_SOFTMAX_ALL selects
 * like MOE_SCORE_SOFTMAX but keeps the selected probabilities of the softmax
 * over all E experts as they are, without renormalising them over the k
 * (the build guide's TopKGate, step 2, as its code is written). */
enum { MOE_SCORE_SOFTMAX = 0, MOE_SCORE_SIGMOID = 1, MOE_SCORE_SOFTMAX_ALL = 2 };

/* Expert FFN kind (see moe_expert_ffn). */
enum { MOE_EXPERT_SILU_MLP = 0, MOE_EXPERT_SWIGLU = 1, MOE_EXPERT_GELU_MLP = 2 };

/* What a (token, expert) pair dropped by the capacity limit contributes to
 * the token's output (see moe_combine): nothing, or the token itself in the
 * pair's slot (Expert Networks, In[10]: a dropped token passes through). */
enum { MOE_DROP_ZERO = 0, MOE_DROP_RESIDUAL = 1 };

#define MOE_MAX_EXPERTS 256

/* ---- problem description ------------------------------------------------ */
typedef struct moe_desc {
    int64_t T;           /* tokens: rows of x (batch x sequence, flattened)   */
    int32_t d_model;     /* token width                                        */
    int32_t d_ff;        /* hidden width of each routed expert                 */
    int32_t E;           /* routed experts, 1..256                             */
    int32_t k;           /* experts per token, 1..E                            */
    int32_t dtype;       /* MOE_F32 or MOE_BF16 (x, expert weights, Y, out)    */
    int32_t score_fn;    /* MOE_SCORE_SOFTMAX, _SIGMOID or _SOFTMAX_ALL        */
    int32_t expert_kind; /* MOE_EXPERT_SILU_MLP, _SWIGLU or _GELU_MLP          */
    int32_t n_shared;    /* 0 or 1 always-on shared expert                     */
    int32_t d_ff_shared; /* hidden width of the shared expert; must equal d_ff */
    int32_t drop_policy; /* MOE_DROP_ZERO (0) or MOE_DROP_RESIDUAL             */
    int64_t capacity;    /* per-expert token limit; < 0 means no limit         */
} moe_desc;

/* ---- parameters (device pointers) --------------------------------------- */
typedef struct moe_weights {
    const void *w_router;     /* [E][d_model] dtype                      required */
    const float *router_bias; /* [E] f32 added to the logits (moves selection
                                 and weights) or NULL                          */
    const float *sel_bias;    /* [E] f32 added to the sigmoid affinity for the
                                 top-k choice only, or NULL; ignored by softmax */
    const void *w_act;        /* [E][d_ff][d_model]  SiLU branch         required */
    const void *w_lin;        /* [E][d_ff][d_model]  linear branch   SwiGLU only */
    const void *w_down;       /* [E][d_model][d_ff]  down projection     required */
    const void *b_act;        /* [E][d_ff]   dtype, SiLU/GELU MLP, NULL = zero;
                                 must be NULL for SwiGLU                        */
    const void *b_down;       /* [E][d_model] dtype, SiLU/GELU MLP, NULL = zero;
                                 must be NULL for SwiGLU                        */
    const void *ws_act;       /* shared expert [d_ff][d_model]  (n_shared = 1)    */
    const void *ws_lin;       /* shared expert [d_ff][d_model]  SwiGLU only       */
    const void *ws_down;      /* shared expert [d_model][d_ff]                    */
    const void *bs_act;       /* shared expert [d_ff], SiLU/GELU MLP, or NULL
                                 (NULL for SwiGLU)                              */
    const void *bs_down;      /* shared expert [d_model], SiLU/GELU MLP, or NULL
                                 (NULL for SwiGLU)                              */
} moe_weights;

/* Optional outputs of moe_forward; any member may be NULL.  The logits are
 * written to memory only when `logits` (or `balance`, which reads them) is
 * set. */
typedef struct moe_forward_aux {
    float *logits;            /* [T][E] f32 gate logits                        */
    int32_t *topk_idx;        /* [T][k] chosen experts, best first              */
    float *topk_w;            /* [T][k] routing weights                         */
    int32_t *counts_assigned; /* [E] pairs routed to each expert before drops   */
    int32_t *counts_kept;     /* [E] pairs each expert processed                */
    int64_t *n_dropped;       /* [1] pairs dropped by the capacity limit        */
    float *balance;           /* [3] balance statistics as moe_balance_stats
                                 writes them; NULL = not computed               */
    float *p_mean;            /* [E] mean router probabilities (needs balance)  */
    float balance_coef;       /* coefficient of the balance loss                */
} moe_forward_aux;

/* ---- host helpers (no GPU work) ----------------------------------------- */

/* Per-expert capacity floor(capacity_factor * T / E), computed in double.
 * capacity_factor <= 0 (or NaN) returns -1 (no limit); E <= 0 or T < 0
 * returns -1.  A limit of T or more -- including an infinite factor -- is
 * returned as T: an expert never receives more than T pairs, so it is the
 * same limit.
 * The build guide gives T * load_factor / E (step 3, apply_capacity) and
 * Expert Networks gives int(cf * (T // E)) (In[10]); they agree whenever E
 * divides T. */
int64_t moe_capacity(int64_t T, int32_t E, double capacity_factor);

/* Routed rows the expert stage may produce: min(T*k, E*capacity) (T*k without
 * a limit).  Y holds these rows first, then T shared-expert rows.  Returns -1
 * for an invalid desc. */
int64_t moe_routed_rows_max(const moe_desc *desc);

/* Bytes of workspace that any entry point below needs for `desc` (the
 * largest, moe_forward's).  Returns 0 for an invalid desc. */
size_t moe_workspace_size(const moe_desc *desc);

/* Static text for a status code. */
const char *moe_status_str(int status);

/* ---- entry points -------------------------------------------------------- */

/* Gate + top-k selection + routing weights.
 * Gate: a linear layer over each token row (build guide step 2 TopKGate;
 * LLMs-from-scratch MoE guide, "Gate computation").  Selection: the k largest
 * scores, ties to the lower expert index, -0 tying with +0.  Softmax routing
 * scores by the logit and weights w_s = exp(l_s) / sum over the selected k of
 * exp(l_j) (LLMs-from-scratch MoE guide, "Top-k selection" and "Routing
 * probabilities"; equal to softmax over all experts renormalised over the
 * top-k, build guide step 2).  MOE_SCORE_SOFTMAX_ALL selects the same way
 * and weights w_s = exp(l_s) / sum over all E experts of exp(l_j).  Sigmoid routing scores by sigmoid(l) +
 * sel_bias and weights by sigmoid(l_s) / sum over the selected of
 * sigmoid(l_j): the bias moves the choice only (DeepSeek 5.7, section 2).
 *
 * Exactly one of x ([T][d_model] dtype) and logits_in ([T][E] f32, the final
 * logits, router_bias already included) must be non-NULL.  With x the gate is
 * computed on the GPU with float32 accumulation; logits_out ([T][E] f32) is
 * optional: when it is NULL the selection runs in the gate's own workgroups
 * and the logits never reach memory, otherwise they are written there too.
 * Either way the indices and weights are the same bits (the gate splits
 * d_model into the same eight ranges, summed in the same order, for every
 * batch size and kernel shape).  With logits_in, weights->w_router may be
 * NULL and logits_out must be NULL.
 * Outputs: topk_idx [T][k] int32 (slot 0 = best), topk_w [T][k] f32. */
int moe_route(const moe_desc *desc, const moe_weights *weights, const void *x,
              const float *logits_in, float *logits_out, int32_t *topk_idx,
              float *topk_w, void *stream);

/* Capacity + dispatch: group the kept (token, expert) pairs by expert.
 * Pairs are visited in token order, then slot order; a pair is kept while its
 * expert has fewer than `capacity` kept pairs (Expert Networks,
 * process_with_capacity in In[10], generalised to k slots); dropped pairs
 * contribute nothing downstream.  Rows are grouped by ascending expert,
 * ascending token within an expert, keeping token identity (DeepSeek 5.7,
 * section 3).
 * Outputs: counts_assigned [E], counts_kept [E], offsets [E+1] (exclusive scan
 * of counts_kept), sorted_token [moe_routed_rows_max] (the first offsets[E]
 * entries are valid), row_of [T][k] (dispatch row of each pair, -1 when
 * dropped), n_dropped [1] int64.  ws: workspace of moe_workspace_size bytes.
 * The debug build returns MOE_ERR_SHAPE (nothing dispatched) when a token row
 * holds an index outside [0, E) or one expert twice. */
int moe_dispatch(const moe_desc *desc, const int32_t *topk_idx, int32_t *counts_assigned,
                 int32_t *counts_kept, int32_t *offsets, int32_t *sorted_token,
                 int32_t *row_of, int64_t *n_dropped, void *ws, size_t ws_bytes,
                 void *stream);

/* The precondition of moe_dispatch on a routing (DeepSeek 5.7, "How do I
 * review an implementation?": check indexing and masks): *n_bad receives the
 * number of token rows of topk_idx [T][k] that hold an index outside [0, E)
 * or one expert twice.  n_bad: one int32 in device memory, written (after
 * being cleared on the stream) when the stream reaches the call; T = 0
 * writes nothing. */
int moe_check_routing(const moe_desc *desc, const int32_t *topk_idx, int32_t *n_bad,
                      void *stream);

/* 1 in the debug build (libmoe_debug.so: moe_dispatch checks its routing
 * with moe_check_routing, synchronises the stream to read the result and
 * returns MOE_ERR_SHAPE on a violation), 0 in the release build. */
int moe_debug_checks(void);

/* Expert FFNs over dispatched rows, plus the shared expert.
 * SiLU MLP: y = W_down (silu(W_act x + b_act)) + b_down (Expert Networks,
 * In[7]).  GELU MLP: y = W_down (gelu(W_act x + b_act)) + b_down with the
 * exact gelu(z) = z/2 (1 + erf(z / sqrt 2)) (build guide step 1, Expert).
 * SwiGLU: y = W_down (silu(W_act x) * (W_lin x)) (LLMs-from-scratch
 * MoE guide, "Expert forward pass"; DeepSeek 5.7, section 1).  Shared expert:
 * the same function with the ws_* weights on every token (DeepSeek 5.7,
 * section 4).
 * Inputs: x [T][d_model]; offsets [E+1] and sorted_token from moe_dispatch.
 * Output Y [moe_routed_rows_max + n_shared*T][d_model] dtype: row r <
 * offsets[E] is the output of the expert owning r for token sorted_token[r];
 * row moe_routed_rows_max + t is the shared expert's output for token t.
 * Other rows are left untouched.  For bf16 the hidden activation is rounded
 * to bf16 between the two projections; accumulation is float32. */
int moe_expert_ffn(const moe_desc *desc, const moe_weights *weights, const void *x,
                   const int32_t *offsets, const int32_t *sorted_token, void *Y,
                   void *ws, size_t ws_bytes, void *stream);

/* Weighted combine: out[t] = sum over slots s with row_of[t][s] >= 0 of
 * topk_w[t][s] * Y[row_of[t][s]], plus Y_shared[t] when Y_shared is not NULL
 * (build guide step 5 combine; LLMs-from-scratch MoE guide, "Weighted
 * aggregation"; DeepSeek 5.7, section 4).  A dropped slot (row_of < 0) adds
 * nothing, or with desc->drop_policy == MOE_DROP_RESIDUAL it adds
 * topk_w[t][s] * x[t]: the token passes through in that slot (Expert
 * Networks, In[10], where a dropped token's output is the token itself).
 * Float32 accumulation in slot order, shared row last; the result is
 * deterministic.  Surviving weights are not renormalised.
 * Y: [moe_routed_rows_max][d_model] dtype; row_of entries are -1 or lie in
 * [0, moe_routed_rows_max) (as moe_dispatch produces them).  Y_shared:
 * [T][d_model] dtype or NULL.  x: [T][d_model] dtype, required with the
 * residual drop policy and ignored otherwise.  out: [T][d_model] dtype. */
int moe_combine(const moe_desc *desc, const void *Y, const void *Y_shared, const void *x,
                const int32_t *row_of, const float *topk_w, void *out, void *stream);

/* Balance statistics of one routing (SNEPPX SER MoE tutorial, step 4
 * "Load-balancing loss"; DeepSeek 5.7, "Implementation and measurement plan":
 * a load histogram and its coefficient of variation).
 *   p_mean[e] = (1/T) sum over tokens of softmax over all E of logits[t]
 *               (in either score mode)
 *   stats[0]  = coef * sum_e (counts_assigned[e] / T) * p_mean[e]
 *   stats[1]  = coefficient of variation of counts_assigned: population
 *               standard deviation over the mean
 *   stats[2]  = max_e counts_assigned[e] / mean
 * logits: [T][E] f32 (moe_route's logits_out); counts_assigned: [E] int32
 * (moe_dispatch's, routes before the capacity limit).  Outputs: stats [3]
 * f32, p_mean [E] f32 or NULL.  Sums run in double in a fixed order: the
 * result is deterministic.  ws: workspace of moe_workspace_size bytes. */
int moe_balance_stats(const moe_desc *desc, const float *logits,
                      const int32_t *counts_assigned, float coef, float *p_mean, float *stats,
                      void *ws, size_t ws_bytes, void *stream);

/* The whole layer: route (from x) -> dispatch -> experts -> combine, on one
 * stream, with no device-to-host copy (a hidden host synchronisation is a
 * failure mode named in DeepSeek 5.7, "Failure modes").
 * x [T][d_model] dtype -> out [T][d_model] dtype.  aux may be NULL; with
 * aux->balance set, the balance statistics of the routing are computed too.
 * ws: workspace of at least moe_workspace_size(desc) bytes. */
int moe_forward(const moe_desc *desc, const moe_weights *weights, const void *x, void *out,
                const moe_forward_aux *aux, void *ws, size_t ws_bytes, void *stream);

/* The whole layer for callers that cannot allocate device memory: code under
 * HIP graph capture, tight serving loops, harnesses that forbid allocation.
 * Same arguments, kernels and results (bit for bit) as moe_forward, but no
 * workspace argument: the library's own scratch array is used instead.  That
 * array is a static device array of moe_scratch_bytes() (64 MiB), one per
 * GPU the library runs on, held until the process ends; its device address
 * is looked up once per device on the first call there.  The call itself
 * allocates and frees nothing.
 *   - Layers whose moe_workspace_size() exceeds moe_scratch_bytes() are
 *     refused with MOE_ERR_TOO_LARGE before anything is enqueued (64 MiB
 *     covers, e.g., a 64-token DeepSeek-V3-shape decode layer, ~11 MB, or a
 *     512-token Qwen3-shape layer, ~25 MB).
 *   - Every call on one GPU shares that GPU's array and leaves its contents
 *     there; nothing in it needs to start at zero (each call writes every
 *     region before reading it).  Calls that overlap on one GPU -- on
 *     different streams, or from different host threads -- race on the array
 *     and must be serialised by the caller.
 *   - Argument errors are reported as by moe_forward, before any HIP call. */
int moe_forward_noalloc(const moe_desc *desc, const moe_weights *weights, const void *x,
                        void *out, const moe_forward_aux *aux, void *stream);

/* Bytes of the static scratch array behind moe_forward_noalloc. */
size_t moe_scratch_bytes(void);

#ifdef __cplusplus
}
#endif
#endif /* MOE_H */
