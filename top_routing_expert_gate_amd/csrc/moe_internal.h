// Internal declarations shared by the HIP translation units of libmoe.
// Not part of the public ABI (include/moe.h is).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "moe.h"

namespace moe {

// ---------------------------------------------------------------------------
// tile height of the f32 grouped GEMM (the bf16 kernel picks its own per call;
// each launcher builds the matching M-tile schedule)
// ---------------------------------------------------------------------------
constexpr int kGemmBMf32 = 64;   // rows per tile of the f32 grouped GEMM
constexpr int kMaxGroups = MOE_MAX_EXPERTS + 1;  // routed experts + shared


// ---------------------------------------------------------------------------
// workspace layout (byte offsets into the caller's workspace)
// ---------------------------------------------------------------------------
struct Workspace {
    size_t topk_idx, topk_w, logits;             // route outputs (forward)
    size_t counts_assigned, counts_kept, offsets; // dispatch outputs (forward)
    size_t sorted_token, row_of, n_dropped;
    size_t chunk_counts;                          // dispatch scratch
    size_t mtile_start;                           // grouped-GEMM schedule
    size_t H;                                     // hidden activations
    size_t Y;                                     // expert outputs (forward)
    size_t balance;                               // balance-statistics partial sums
    size_t check;                                 // routing-check counter (debug builds)
    size_t total;
    int64_t rows_routed_max;  // routed rows of H / Y
    int64_t rows_total;       // + n_shared * T
    int chunk_tokens, n_chunks;
    int bal_rows, bal_blocks;  // token rows per partial-sum block, and blocks
};

// Bytes of the static scratch array behind moe_forward_noalloc (per GPU).
constexpr size_t kScratchBytes = (size_t)64 << 20;
// Device address of that array on the current GPU (looked up once per device).
int scratch_address(void **ptr);
// moe_forward on a given workspace.
int forward_impl(const moe_desc *desc, const moe_weights *weights, const void *x, void *out,
                 const moe_forward_aux *aux, void *ws, size_t ws_bytes, void *stream);

// Returns false for an invalid desc.
bool workspace_layout(const moe_desc &d, Workspace *w);
int validate_desc(const moe_desc &d);
// min(T*k, E*capacity), or T*k without a limit (no overflow for any capacity)
int64_t routed_rows(const moe_desc &d);

inline int elem_bytes(int dtype) { return dtype == MOE_BF16 ? 2 : 4; }
inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

// ---------------------------------------------------------------------------
// launchers (each returns hipSuccess or the launch error)
// ---------------------------------------------------------------------------

// K1: gate + top-k.  logits: where the caller wants the f32 logits, or NULL;
// logits_buf: a buffer the gate may use when a separate top-k launch is
// faster (NULL: the selection is fused into the gate).  The logits, indices
// and weights are the same bits whichever kernels run.  chunk_counts (or
// NULL): when the selection runs fused and route_chunk_tokens(d) > 0, the
// per-chunk expert counts of the dispatch walk for chunks of that many
// tokens ([n_chunks][E]), as dispatch_count_kernel would write them.
hipError_t launch_route(const moe_desc &d, const void *x, const void *w_router,
                        const float *router_bias, const float *sel_bias, float *logits,
                        float *logits_buf, int32_t *topk_idx, float *topk_w, hipStream_t s,
                        int32_t *chunk_counts = nullptr);

// Tokens per gate block when the route runs gate and selection in one launch
// with the given buffers' layout (bf16 layers whose router is small), else 0:
// the dispatch chunk for which that launch can count the experts.
int route_chunk_tokens(const moe_desc &d);

// K1, selection only: top-k + routing weights from f32 logits.
hipError_t launch_topk(const moe_desc &d, const float *logits, const float *sel_bias,
                       int32_t *topk_idx, float *topk_w, hipStream_t s);

// K2: capacity + dispatch (three kernels).  schedule_bm > 0 also writes the
// grouped-GEMM M-tile schedule for tiles of that many rows into the workspace.
// counts_ready: the per-chunk expert counts are already in the workspace (the
// fused route wrote them), so the counting kernel is skipped.
hipError_t launch_dispatch(const moe_desc &d, const Workspace &w, const int32_t *topk_idx,
                           int32_t *counts_assigned, int32_t *counts_kept, int32_t *offsets,
                           int32_t *sorted_token, int32_t *row_of, int64_t *n_dropped,
                           char *ws, hipStream_t s, int schedule_bm = 0,
                           bool counts_ready = false);

// Rows of topk_idx [T][k] holding an index outside [0, E) or one expert
// twice, counted into n_bad (device int, cleared first by a kernel).
hipError_t launch_check_routing(const moe_desc &d, const int32_t *topk_idx, int32_t *n_bad,
                                hipStream_t s);

// K3: grouped expert FFN (schedule + up projection + down projection).
struct ExpertArgs {
    const void *x;
    const int32_t *offsets;
    const int32_t *sorted_token;
    void *Y;
    char *ws;
};
hipError_t launch_expert_ffn(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                             const ExpertArgs &a, hipStream_t s);

// Rows per M tile the grouped expert GEMM will use for this layer, and the
// two launchers; with schedule_ready the M-tile schedule is already in the
// workspace (built by the dispatch scan for that tile height).
int grouped_ffn_bm(const moe_desc &d, const Workspace &w);
hipError_t launch_grouped_ffn_bf16(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                                   const ExpertArgs &a, hipStream_t s, bool schedule_ready);
hipError_t launch_grouped_ffn_f32(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                                  const ExpertArgs &a, hipStream_t s, bool schedule_ready);

// K4: weighted combine (+ shared expert row; x for residual drops).
hipError_t launch_combine(const moe_desc &d, const void *Y, const void *Y_shared, const void *x,
                          const int32_t *row_of, const float *topk_w, void *out,
                          hipStream_t s);

// Balance statistics: mean router probabilities, loss, spread of the loads.
hipError_t launch_balance(const moe_desc &d, const Workspace &w, const float *logits,
                          const int32_t *counts_assigned, float coef, float *p_mean,
                          float *stats, char *ws, hipStream_t s);

}  // namespace moe
