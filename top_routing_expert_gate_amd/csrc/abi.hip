// C ABI of libmoe: argument validation, workspace layout and the stage
// sequence of the layer.  Every argument check happens on the host before
// any HIP call, so invalid calls return a status without touching the GPU.
#include <algorithm>
#include <mutex>

#include "moe_internal.h"

namespace moe {

// Routed rows of one call: min(T*k, E*capacity), T*k without a limit.  The
// capacity is clamped to T*k first (an expert never receives more pairs), so
// the product cannot overflow for any capacity a caller passes.
int64_t routed_rows(const moe_desc &d) {
    const int64_t Tk = d.T * d.k;
    if (d.capacity < 0) return Tk;
    return std::min<int64_t>(Tk, (int64_t)d.E * std::min<int64_t>(d.capacity, Tk));
}

int validate_desc(const moe_desc &d) {
    if (d.dtype != MOE_F32 && d.dtype != MOE_BF16) return MOE_ERR_UNSUPPORTED;
    if (d.score_fn != MOE_SCORE_SOFTMAX && d.score_fn != MOE_SCORE_SIGMOID &&
        d.score_fn != MOE_SCORE_SOFTMAX_ALL)
        return MOE_ERR_UNSUPPORTED;
    if (d.expert_kind != MOE_EXPERT_SILU_MLP && d.expert_kind != MOE_EXPERT_SWIGLU &&
        d.expert_kind != MOE_EXPERT_GELU_MLP)
        return MOE_ERR_UNSUPPORTED;
    if (d.drop_policy != MOE_DROP_ZERO && d.drop_policy != MOE_DROP_RESIDUAL)
        return MOE_ERR_UNSUPPORTED;
    if (d.E > MOE_MAX_EXPERTS) return MOE_ERR_UNSUPPORTED;
    if (d.T < 0 || d.E < 1 || d.k < 1 || d.k > d.E) return MOE_ERR_SHAPE;
    if (d.d_model < 8 || d.d_model % 8 != 0 || d.d_ff < 8 || d.d_ff % 8 != 0) return MOE_ERR_SHAPE;
    if (d.n_shared != 0 && d.n_shared != 1) return MOE_ERR_SHAPE;
    if (d.n_shared == 1 && d.d_ff_shared != d.d_ff) return MOE_ERR_SHAPE;
    // 32-bit row indices inside the kernels
    if (d.T * (int64_t)d.k > INT32_MAX || d.T > INT32_MAX / 2) return MOE_ERR_SHAPE;
    // the operands the kernels address with 32-bit byte offsets from one base
    // stay below 2 GiB: x (its rows are gathered from anywhere in it), one
    // expert's matrix and the router.  H and Y are addressed per tile or per
    // row and may be larger.
    const int64_t es = elem_bytes(d.dtype);
    const int64_t lim = (int64_t)INT32_MAX;
    if (d.T * d.d_model * es > lim || (int64_t)d.d_ff * d.d_model * es > lim ||
        (int64_t)d.E * d.d_model * es > lim)
        return MOE_ERR_SHAPE;
    return MOE_OK;
}

static size_t align_up(size_t v) { return (v + 255) & ~size_t(255); }

bool workspace_layout(const moe_desc &d, Workspace *w) {
    if (validate_desc(d) != MOE_OK) return false;
    const int64_t Tk = d.T * d.k;
    w->rows_routed_max = routed_rows(d);
    w->rows_total = w->rows_routed_max + (int64_t)d.n_shared * d.T;
    // chunks of the dispatch walk: at least 64 tokens, at most 2048 chunks;
    // where the route fuses gate and selection, its blocks' rows instead (if
    // that still makes at most 2048 chunks), so that the route can count the
    // experts per chunk and the counting launch is skipped
    w->chunk_tokens = (int)std::max<int64_t>(64, ceil_div(std::max<int64_t>(d.T, 1), 2048));
    const int rct = route_chunk_tokens(d);
    if (rct > 0 && ceil_div(d.T, rct) <= 2048) w->chunk_tokens = rct;
    w->n_chunks = (int)ceil_div(d.T, w->chunk_tokens);
    // balance statistics: at least 64 token rows per partial sum, at most 1024 sums
    w->bal_rows = (int)std::max<int64_t>(64, ceil_div(std::max<int64_t>(d.T, 1), 1024));
    w->bal_blocks = (int)ceil_div(d.T, w->bal_rows);
    const int es = elem_bytes(d.dtype);
    const int G = d.E + d.n_shared;
    size_t o = 0;
    w->logits = o;          o = align_up(o + (size_t)d.T * d.E * 4);
    w->topk_idx = o;        o = align_up(o + (size_t)Tk * 4);
    w->topk_w = o;          o = align_up(o + (size_t)Tk * 4);
    w->counts_assigned = o; o = align_up(o + (size_t)d.E * 4);
    w->counts_kept = o;     o = align_up(o + (size_t)d.E * 4);
    w->offsets = o;         o = align_up(o + (size_t)(d.E + 1) * 4);
    w->n_dropped = o;       o = align_up(o + 8);
    w->sorted_token = o;    o = align_up(o + (size_t)w->rows_routed_max * 4);
    w->row_of = o;          o = align_up(o + (size_t)Tk * 4);
    w->chunk_counts = o;    o = align_up(o + (size_t)w->n_chunks * d.E * 4);
    w->mtile_start = o;     o = align_up(o + (size_t)(G + 1) * 4);
    w->H = o;               o = align_up(o + (size_t)w->rows_total * d.d_ff * es);
    w->Y = o;               o = align_up(o + (size_t)w->rows_total * d.d_model * es);
    w->balance = o;         o = align_up(o + (size_t)w->bal_blocks * d.E * 8);
    w->check = o;           o = align_up(o + 4);
    w->total = o;
    return true;
}

static int check_weights_experts(const moe_desc &d, const moe_weights *wt) {
    if (!wt || !wt->w_act || !wt->w_down) return MOE_ERR_NULL;
    if (d.expert_kind == MOE_EXPERT_SWIGLU && !wt->w_lin) return MOE_ERR_NULL;
    // the SwiGLU expert has no biases: refuse them rather than ignore them
    if (d.expert_kind == MOE_EXPERT_SWIGLU &&
        (wt->b_act || wt->b_down || wt->bs_act || wt->bs_down))
        return MOE_ERR_UNSUPPORTED;
    if (d.n_shared) {
        if (!wt->ws_act || !wt->ws_down) return MOE_ERR_NULL;
        if (d.expert_kind == MOE_EXPERT_SWIGLU && !wt->ws_lin) return MOE_ERR_NULL;
    }
    return MOE_OK;
}

static int hip_status(hipError_t e) { return e == hipSuccess ? MOE_OK : MOE_ERR_HIP; }

static hipError_t expert_ffn(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                             const ExpertArgs &a, hipStream_t s, bool schedule_ready) {
    return d.dtype == MOE_BF16 ? launch_grouped_ffn_bf16(d, wt, w, a, s, schedule_ready)
                               : launch_grouped_ffn_f32(d, wt, w, a, s, schedule_ready);
}

// Scratch for moe_forward_noalloc: one array per GPU the library runs on,
// held until the process ends.  In host code `scratch` names a host-side
// stand-in, not device memory: its device address on the current GPU comes
// from hipGetSymbolAddress, once per device, and only that address is ever
// handed to kernels.
static __device__ __align__(256) unsigned char scratch[kScratchBytes];

constexpr int kMaxDevices = 64;
static void *g_scratch_ptr[kMaxDevices];
static std::mutex g_scratch_mu;

int scratch_address(void **ptr) {
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) return MOE_ERR_HIP;
    std::lock_guard<std::mutex> lock(g_scratch_mu);
    if (!g_scratch_ptr[dev]) {
        void *p = nullptr;
        if (hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)) != hipSuccess || !p) return MOE_ERR_HIP;
        g_scratch_ptr[dev] = p;
    }
    *ptr = g_scratch_ptr[dev];
    return MOE_OK;
}

}  // namespace moe

using namespace moe;

extern "C" {

int64_t moe_capacity(int64_t T, int32_t E, double capacity_factor) {
    if (!(capacity_factor > 0.0) || E <= 0 || T < 0) return -1;
    const double c = capacity_factor * (double)T / (double)E;
    // an expert never receives more than T pairs: any larger limit (or an
    // infinite factor) is the same as T, and the conversion stays in range
    if (!(c < (double)T)) return T;
    return (int64_t)c;  // floor for 0 <= c < T
}

int64_t moe_routed_rows_max(const moe_desc *desc) {
    Workspace w;
    if (!desc || !workspace_layout(*desc, &w)) return -1;
    return w.rows_routed_max;
}

size_t moe_workspace_size(const moe_desc *desc) {
    Workspace w;
    if (!desc || !workspace_layout(*desc, &w)) return 0;
    return w.total;
}

const char *moe_status_str(int status) {
    switch (status) {
        case MOE_OK: return "ok";
        case MOE_ERR_NULL: return "a required pointer is NULL";
        case MOE_ERR_SHAPE: return "invalid shape (T, E, k, d_model, d_ff or shared width)";
        case MOE_ERR_UNSUPPORTED:
            return "unsupported (E > 256, dtype, score function, expert kind or drop policy)";
        case MOE_ERR_WORKSPACE: return "workspace smaller than moe_workspace_size()";
        case MOE_ERR_HIP: return "HIP launch failed";
        case MOE_ERR_TOO_LARGE:
            return "the layer needs more scratch than moe_forward_noalloc's static array "
                   "(moe_scratch_bytes()): use moe_forward with a workspace";
        default: return "unknown status";
    }
}

int moe_route(const moe_desc *desc, const moe_weights *weights, const void *x,
              const float *logits_in, float *logits_out, int32_t *topk_idx, float *topk_w,
              void *stream) {
    if (!desc || !topk_idx || !topk_w) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    if ((x == nullptr) == (logits_in == nullptr)) return MOE_ERR_NULL;
    if (logits_in && logits_out) return MOE_ERR_SHAPE;
    if (x && (!weights || !weights->w_router)) return MOE_ERR_NULL;
    if (desc->T == 0) return MOE_OK;
    hipStream_t s = (hipStream_t)stream;
    const moe_desc &d = *desc;
    const float *sel_bias = weights ? weights->sel_bias : nullptr;
    if (x)  // logits_out may be NULL: the selection then runs inside the gate
        return hip_status(launch_route(d, x, weights->w_router, weights->router_bias, sel_bias,
                                       logits_out, logits_out, topk_idx, topk_w, s));
    return hip_status(launch_topk(d, logits_in, sel_bias, topk_idx, topk_w, s));
}

int moe_dispatch(const moe_desc *desc, const int32_t *topk_idx, int32_t *counts_assigned,
                 int32_t *counts_kept, int32_t *offsets, int32_t *sorted_token, int32_t *row_of,
                 int64_t *n_dropped, void *ws, size_t ws_bytes, void *stream) {
    if (!desc || !topk_idx || !counts_assigned || !counts_kept || !offsets || !sorted_token ||
        !row_of || !n_dropped || !ws)
        return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    Workspace w;
    workspace_layout(*desc, &w);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
    if (desc->T == 0) return MOE_OK;
#ifdef MOE_DEBUG_CHECKS
    // debug builds check the routing first (and synchronise the stream to
    // read the result): MOE_ERR_SHAPE if a row breaks the precondition
    {
        int32_t *n_bad = (int32_t *)((char *)ws + w.check);
        if (launch_check_routing(*desc, topk_idx, n_bad, (hipStream_t)stream) != hipSuccess)
            return MOE_ERR_HIP;
        int32_t bad = 0;
        if (hipMemcpyAsync(&bad, n_bad, sizeof(bad), hipMemcpyDeviceToHost,
                           (hipStream_t)stream) != hipSuccess ||
            hipStreamSynchronize((hipStream_t)stream) != hipSuccess)
            return MOE_ERR_HIP;
        if (bad) return MOE_ERR_SHAPE;
    }
#endif
    return hip_status(launch_dispatch(*desc, w, topk_idx, counts_assigned, counts_kept, offsets,
                                      sorted_token, row_of, n_dropped, (char *)ws,
                                      (hipStream_t)stream));
}

int moe_expert_ffn(const moe_desc *desc, const moe_weights *weights, const void *x,
                   const int32_t *offsets, const int32_t *sorted_token, void *Y, void *ws,
                   size_t ws_bytes, void *stream) {
    if (!desc || !x || !offsets || !sorted_token || !Y || !ws) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    st = check_weights_experts(*desc, weights);
    if (st != MOE_OK) return st;
    Workspace w;
    workspace_layout(*desc, &w);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
    if (desc->T == 0) return MOE_OK;
    ExpertArgs a{x, offsets, sorted_token, Y, (char *)ws};
    return hip_status(expert_ffn(*desc, *weights, w, a, (hipStream_t)stream, false));
}

int moe_combine(const moe_desc *desc, const void *Y, const void *Y_shared, const void *x,
                const int32_t *row_of, const float *topk_w, void *out, void *stream) {
    if (!desc || !Y || !row_of || !topk_w || !out) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    if (desc->drop_policy == MOE_DROP_RESIDUAL && !x) return MOE_ERR_NULL;
    if (desc->T == 0) return MOE_OK;
    return hip_status(launch_combine(*desc, Y, Y_shared, x, row_of, topk_w, out,
                                     (hipStream_t)stream));
}

int moe_check_routing(const moe_desc *desc, const int32_t *topk_idx, int32_t *n_bad,
                      void *stream) {
    if (!desc || !topk_idx || !n_bad) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    return hip_status(launch_check_routing(*desc, topk_idx, n_bad, (hipStream_t)stream));
}

int moe_debug_checks(void) {
#ifdef MOE_DEBUG_CHECKS
    return 1;
#else
    return 0;
#endif
}

int moe_balance_stats(const moe_desc *desc, const float *logits, const int32_t *counts_assigned,
                      float coef, float *p_mean, float *stats, void *ws, size_t ws_bytes,
                      void *stream) {
    if (!desc || !logits || !counts_assigned || !stats || !ws) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    Workspace w;
    workspace_layout(*desc, &w);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
    if (desc->T == 0) return MOE_OK;
    return hip_status(launch_balance(*desc, w, logits, counts_assigned, coef, p_mean, stats,
                                     (char *)ws, (hipStream_t)stream));
}

int moe_forward(const moe_desc *desc, const moe_weights *weights, const void *x, void *out,
                const moe_forward_aux *aux, void *ws, size_t ws_bytes, void *stream) {
    return moe::forward_impl(desc, weights, x, out, aux, ws, ws_bytes, stream);
}

size_t moe_scratch_bytes(void) { return moe::kScratchBytes; }

int moe_forward_noalloc(const moe_desc *desc, const moe_weights *weights, const void *x,
                        void *out, const moe_forward_aux *aux, void *stream) {
    // every check of moe_forward first, so that a refused call touches no GPU
    if (!desc || !weights || !x || !out) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    if (!weights->w_router) return MOE_ERR_NULL;
    st = check_weights_experts(*desc, weights);
    if (st != MOE_OK) return st;
    if (desc->T == 0) return MOE_OK;
    Workspace w;
    workspace_layout(*desc, &w);
    if (w.total > kScratchBytes) return MOE_ERR_TOO_LARGE;
    void *ptr = nullptr;
    st = moe::scratch_address(&ptr);
    if (st != MOE_OK) return st;
    return moe::forward_impl(desc, weights, x, out, aux, ptr, kScratchBytes, stream);
}

}  // extern "C"

namespace moe {

int forward_impl(const moe_desc *desc, const moe_weights *weights, const void *x, void *out,
                 const moe_forward_aux *aux, void *ws, size_t ws_bytes, void *stream) {
    if (!desc || !weights || !x || !out || !ws) return MOE_ERR_NULL;
    int st = validate_desc(*desc);
    if (st != MOE_OK) return st;
    if (!weights->w_router) return MOE_ERR_NULL;
    st = check_weights_experts(*desc, weights);
    if (st != MOE_OK) return st;
    Workspace w;
    workspace_layout(*desc, &w);
    if (ws_bytes < w.total) return MOE_ERR_WORKSPACE;
    if (desc->T == 0) return MOE_OK;
    const moe_desc &d = *desc;
    hipStream_t s = (hipStream_t)stream;
    char *b = (char *)ws;
    moe_forward_aux none{};
    const moe_forward_aux &ax = aux ? *aux : none;
    // logits reach memory only when the caller or the balance statistics read
    // them; the workspace copy also serves a separate top-k launch
    float *logits_ws = (float *)(b + w.logits);
    float *logits = ax.logits ? ax.logits : ax.balance ? logits_ws : nullptr;
    int32_t *topk_idx = ax.topk_idx ? ax.topk_idx : (int32_t *)(b + w.topk_idx);
    float *topk_w = ax.topk_w ? ax.topk_w : (float *)(b + w.topk_w);
    int32_t *ca = ax.counts_assigned ? ax.counts_assigned : (int32_t *)(b + w.counts_assigned);
    int32_t *ck = ax.counts_kept ? ax.counts_kept : (int32_t *)(b + w.counts_kept);
    int64_t *nd = ax.n_dropped ? ax.n_dropped : (int64_t *)(b + w.n_dropped);
    int32_t *offsets = (int32_t *)(b + w.offsets);
    int32_t *sorted_token = (int32_t *)(b + w.sorted_token);
    int32_t *row_of = (int32_t *)(b + w.row_of);
    void *Y = b + w.Y;

    // where the route fuses gate and selection with blocks of one dispatch
    // chunk, it also counts the experts per chunk
    const bool counted = route_chunk_tokens(d) == w.chunk_tokens;
    int32_t *chunk_counts = counted ? (int32_t *)(b + w.chunk_counts) : nullptr;
    hipError_t e = launch_route(d, x, weights->w_router, weights->router_bias, weights->sel_bias,
                                logits, logits ? logits : logits_ws, topk_idx, topk_w, s,
                                chunk_counts);
    // the dispatch scan also lays out the expert GEMM's tile schedule
    if (e == hipSuccess)
        e = launch_dispatch(d, w, topk_idx, ca, ck, offsets, sorted_token, row_of, nd, b, s,
                            grouped_ffn_bm(d, w), counted);
    if (e == hipSuccess) {
        ExpertArgs a{x, offsets, sorted_token, Y, b};
        e = expert_ffn(d, *weights, w, a, s, true);
    }
    if (e == hipSuccess) {
        const void *Ys = d.n_shared
                             ? (const void *)((char *)Y + (size_t)w.rows_routed_max * d.d_model *
                                                              elem_bytes(d.dtype))
                             : nullptr;
        e = launch_combine(d, Y, Ys, x, row_of, topk_w, out, s);
    }
    if (e == hipSuccess && ax.balance)
        e = launch_balance(d, w, logits, ca, ax.balance_coef, ax.p_mean, ax.balance, b, s);
    return hip_status(e);
}

}  // namespace moe
