// K2: capacity + dispatch for gfx950, integer-only and deterministic.
//
// Semantics (Expert Networks > Code Implementation, In[10]
// process_with_capacity, generalised to k slots; DeepSeek 5.7, section 3):
// the (token, slot) pairs are visited in token order then slot order and a
// pair is kept while its expert has fewer than `capacity` kept pairs.  Since a
// token's k experts are distinct, the kept pairs of expert e are exactly its
// first `capacity` tokens in ascending token order, so the sequential walk
// becomes a stable counting sort:
//
//   count   one workgroup per chunk of tokens: per-expert histogram in LDS
//   scan    one workgroup: per-expert exclusive scan over chunks, counts,
//           capped counts, offsets (a workgroup-wide shuffle scan over
//           experts), drop count
//   scatter one wavefront per chunk: walks its pairs in order, 64 at a time
//           (the expert indices of 8 such slabs are loaded together);
//           equal-expert lanes are found with 8 ballots over the expert
//           index bits, a lane's rank is the popcount of equal lanes below
//           it, and the global rank decides keep/drop
//   fused   scan and scatter in one launch where the chunk-count matrix is
//           small: each chunk's workgroup sums the matrix itself (totals,
//           and the chunks before its own), then scatters as above
//
// An index outside [0, E) never reaches memory as an address: count and
// scatter drop its pair (row_of = -1, not counted).  check_routing_kernel
// counts the rows that break the precondition (moe_check_routing, and
// moe_dispatch itself in a debug build).
//
// The grouped-GEMM schedule (M tiles per group, prefix over groups) is
// produced by the scan (or fused) kernel when the whole layer runs
// (moe_forward), or by a one-workgroup kernel when the expert stage is called
// on its own.
#include "moe_internal.h"

namespace moe {
namespace {

// Exclusive prefix sum of one int per thread over the workgroup (at most 16
// wavefronts): a shuffle scan inside each wavefront, then the wavefront
// totals from LDS.  Integer sums, so the result does not depend on order.
// Every thread of the workgroup must call it; `total` is the sum of all.
__device__ __forceinline__ int block_exclusive_scan(int v, int *s_wave, int &total) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, nw = blockDim.x >> 6;
    int x = v;
#pragma unroll
    for (int o = 1; o < 64; o <<= 1) {
        const int y = __shfl_up(x, o);
        if (lane >= o) x += y;
    }
    if (lane == 63) s_wave[wave] = x;
    __syncthreads();
    int base = 0, all = 0;
    for (int q = 0; q < nw; ++q) {
        const int t = s_wave[q];
        base += q < wave ? t : 0;
        all += t;
    }
    __syncthreads();  // s_wave may be reused by the next call
    total = all;
    return base + x - v;
}

__global__ __launch_bounds__(256) void dispatch_count_kernel(
    const int32_t *__restrict__ idx, int32_t *__restrict__ chunk_counts, int64_t T, int k,
    int E, int chunk_tokens) {
    __shared__ int hist[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    __syncthreads();
    const int64_t t0 = (int64_t)blockIdx.x * chunk_tokens;
    const int64_t t1 = min(T, t0 + chunk_tokens);
    for (int64_t i = t0 * k + threadIdx.x; i < t1 * k; i += blockDim.x) {
        const int e = idx[i];
        if ((unsigned)e < (unsigned)E) atomicAdd(&hist[e], 1);  // others: dropped, not counted
    }
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x)
        chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
}

// One workgroup of 1024 threads.  chunk_counts is rewritten in place into the
// per-chunk base rank of each expert.  Each expert's chunks are split into P
// contiguous parts scanned by P threads (P = 1024 / E), then the part sums
// are scanned in LDS.  With mtile_start != NULL the grouped-GEMM M-tile
// schedule for tiles of bm rows is produced as well (group E, when present,
// is the shared expert with T rows).
__global__ __launch_bounds__(1024) void dispatch_scan_kernel(
    int32_t *__restrict__ chunk_counts, int n_chunks, int E, int64_t T, int k, int64_t cap,
    int32_t *__restrict__ counts_assigned, int32_t *__restrict__ counts_kept,
    int32_t *__restrict__ offsets, int64_t *__restrict__ n_dropped,
    int32_t *__restrict__ mtile_start, int bm, int n_shared) {
    __shared__ int part_sum[1024];
    __shared__ int kept_s[MOE_MAX_EXPERTS];
    const int tid = threadIdx.x;
    const int P = 1024 / E;  // threads per expert
    const int e = tid % E, p = tid / E;
    const bool active = p < P;
    const int cs = (n_chunks + P - 1) / P;  // chunks per part
    const int c0 = min(n_chunks, p * cs), c1 = min(n_chunks, c0 + cs);
    int sum = 0;
    if (active) {
        constexpr int kBatch = 16;  // loads in flight per thread
        for (int c = c0; c < c1; c += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = c + j < c1 ? chunk_counts[(int64_t)(c + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) sum += v[j];
        }
        part_sum[p * E + e] = sum;
    }
    __syncthreads();
    if (active) {
        int base = 0, total = 0;
        for (int q = 0; q < P; ++q) {
            const int v = part_sum[q * E + e];
            base += q < p ? v : 0;
            total += v;
        }
        // rewrite this part's chunk counts as running bases
        constexpr int kBatch = 16;
        int run = base;
        for (int c = c0; c < c1; c += kBatch) {
            int v[kBatch];
#pragma unroll
            for (int j = 0; j < kBatch; ++j)
                v[j] = c + j < c1 ? chunk_counts[(int64_t)(c + j) * E + e] : 0;
#pragma unroll
            for (int j = 0; j < kBatch; ++j) {
                if (c + j < c1) chunk_counts[(int64_t)(c + j) * E + e] = run;
                run += v[j];
            }
        }
        if (p == 0) {
            counts_assigned[e] = total;
            const int kept = (cap < 0 || total <= cap) ? total : (int)cap;
            counts_kept[e] = kept;
            kept_s[e] = kept;
        }
    }
    __syncthreads();
    // offsets = exclusive scan of kept over experts; then the tile schedule,
    // an exclusive scan of ceil(rows / bm) over the groups (E <= 256 < 1024
    // threads: one value per thread)
    __shared__ int s_wave[16];
    const int kv = tid < E ? kept_s[tid] : 0;
    int kept_total;
    const int ofs = block_exclusive_scan(kv, s_wave, kept_total);
    if (tid < E) offsets[tid] = ofs;
    if (tid == 0) {
        offsets[E] = kept_total;
        *n_dropped = T * (int64_t)k - kept_total;
    }
    if (mtile_start) {
        const int G = E + n_shared;
        const int tv = tid < E ? (kv + bm - 1) / bm : tid < G ? (int)((T + bm - 1) / bm) : 0;
        int tiles_total;
        const int ts = block_exclusive_scan(tv, s_wave, tiles_total);
        if (tid < G) mtile_start[tid] = ts;
        if (tid == 0) mtile_start[G] = tiles_total;
    }
}

// Walks one chunk's (token, slot) pairs [i0, i1) in order, 64 at a time, on
// wavefront 0 of the workgroup; every thread of the workgroup calls it (the
// slab loop's bounds are uniform) for the barriers.  cnt holds the chunk's
// base rank per expert and is advanced in place; off holds the experts'
// row offsets.
__device__ __forceinline__ void scatter_chunk(const int32_t *__restrict__ idx, int *cnt,
                                              const int *off, int32_t *__restrict__ sorted_token,
                                              int32_t *__restrict__ row_of, int64_t i0,
                                              int64_t i1, int k, int E, int64_t cap, int nbits) {
    const int lane = threadIdx.x & 63;
    const bool worker = threadIdx.x < 64;
    const uint64_t below = (1ull << lane) - 1ull;
    constexpr int kBatch = 8;  // slabs of 64 pairs whose indices are loaded together
    for (int64_t b0 = i0; b0 < i1; b0 += 64 * kBatch) {
        int ev[kBatch];
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t i = b0 + u * 64 + lane;
            ev[u] = worker && i < i1 ? idx[i] : 0;
        }
#pragma unroll
        for (int u = 0; u < kBatch; ++u) {
            const int64_t base = b0 + u * 64;
            if (base >= i1) break;
            if (worker) {
                const int64_t i = base + lane;
                const int e = ev[u];
                const bool in = i < i1;
                const bool ok = in && (unsigned)e < (unsigned)E;  // outside [0, E): dropped
                uint64_t same = __ballot(ok);
                for (int b = 0; b < nbits; ++b) {
                    const bool bit = (e >> b) & 1;
                    const uint64_t m = __ballot(bit);
                    same &= bit ? m : ~m;
                }
                const int rank = __popcll(same & below);
                const int c = ok ? cnt[e] : 0;  // every lane reads before any lane writes
                const int p = c + rank;
                // the highest lane of each equal-expert set advances the counter
                if (ok && (same >> lane) == 1ull) cnt[e] = p + 1;
                if (ok && (cap < 0 || p < cap)) {
                    const int r = off[e] + p;
                    row_of[i] = r;
                    sorted_token[r] = (int32_t)(i / k);
                } else if (in) {
                    row_of[i] = -1;
                }
            }
            __syncthreads();  // orders this slab's counter writes before the next slab's reads
        }
    }
}

// One wavefront (64 threads) per chunk, after dispatch_scan_kernel.
__global__ __launch_bounds__(64) void dispatch_scatter_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ chunk_base,
    const int32_t *__restrict__ offsets, int32_t *__restrict__ sorted_token,
    int32_t *__restrict__ row_of, int64_t T, int k, int E, int64_t cap, int chunk_tokens,
    int nbits) {
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int off[MOE_MAX_EXPERTS];
    for (int e = threadIdx.x; e < E; e += 64) {
        cnt[e] = chunk_base[(int64_t)blockIdx.x * E + e];
        off[e] = offsets[e];
    }
    __syncthreads();
    const int64_t i0 = (int64_t)blockIdx.x * chunk_tokens * k;
    const int64_t i1 = min(T, (int64_t)(blockIdx.x + 1) * chunk_tokens) * k;
    scatter_chunk(idx, cnt, off, sorted_token, row_of, i0, i1, k, E, cap, nbits);
}

// Scan and scatter in one launch, where each of the P = 1024 / E parts of an
// expert's chunks holds at most kFusedPartChunks chunks.  Every workgroup (one
// per chunk) sums the whole chunk-count matrix, kept in registers: the
// experts' totals, and the chunks before its own (its base ranks).  So no
// workgroup waits for another, and chunk_counts is only read.  Workgroup 0
// also writes the counts, offsets, drop count and the M-tile schedule.  The
// sums are integer, so every output has the bits of the scan + scatter pair.
constexpr int kFusedPartChunks = 32;

__global__ __launch_bounds__(1024) void dispatch_fused_kernel(
    const int32_t *__restrict__ idx, const int32_t *__restrict__ chunk_counts, int n_chunks,
    int E, int64_t T, int k, int64_t cap, int32_t *__restrict__ counts_assigned,
    int32_t *__restrict__ counts_kept, int32_t *__restrict__ offsets,
    int64_t *__restrict__ n_dropped, int32_t *__restrict__ mtile_start, int bm, int n_shared,
    int32_t *__restrict__ sorted_token, int32_t *__restrict__ row_of, int chunk_tokens,
    int nbits) {
    __shared__ int pre_s[1024];
    __shared__ int tot_s[1024];
    __shared__ int cnt[MOE_MAX_EXPERTS];
    __shared__ int off[MOE_MAX_EXPERTS];
    __shared__ int s_wave[16];
    const int tid = threadIdx.x;
    const int chunk = blockIdx.x;
    const int P = 1024 / E;  // threads per expert
    const int e = tid % E, p = tid / E;
    const int cs = (n_chunks + P - 1) / P;  // chunks per part, at most kFusedPartChunks
    const int c0 = min(n_chunks, p * cs), c1 = min(n_chunks, c0 + cs);
    if (p < P) {
        int v[kFusedPartChunks];
#pragma unroll
        for (int j = 0; j < kFusedPartChunks; ++j)
            v[j] = c0 + j < c1 ? chunk_counts[(int64_t)(c0 + j) * E + e] : 0;
        int pre = 0, tot = 0;
#pragma unroll
        for (int j = 0; j < kFusedPartChunks; ++j) {
            pre += c0 + j < chunk ? v[j] : 0;
            tot += v[j];
        }
        pre_s[tid] = pre;
        tot_s[tid] = tot;
    }
    __syncthreads();
    int base = 0, total = 0, kv = 0;
    if (tid < E) {
        for (int q = 0; q < P; ++q) {
            base += pre_s[q * E + tid];
            total += tot_s[q * E + tid];
        }
        kv = (cap < 0 || total <= cap) ? total : (int)cap;
    }
    int kept_total;
    const int ofs = block_exclusive_scan(kv, s_wave, kept_total);
    if (tid < E) {
        cnt[tid] = base;
        off[tid] = ofs;
    }
    if (chunk == 0) {
        if (tid < E) {
            counts_assigned[tid] = total;
            counts_kept[tid] = kv;
            offsets[tid] = ofs;
        }
        if (tid == 0) {
            offsets[E] = kept_total;
            *n_dropped = T * (int64_t)k - kept_total;
        }
        if (mtile_start) {
            const int G = E + n_shared;
            const int tv = tid < E ? (kv + bm - 1) / bm : tid < G ? (int)((T + bm - 1) / bm) : 0;
            int tiles_total;
            const int ts = block_exclusive_scan(tv, s_wave, tiles_total);
            if (tid < G) mtile_start[tid] = ts;
            if (tid == 0) mtile_start[G] = tiles_total;
        }
    }
    __syncthreads();
    const int64_t i0 = (int64_t)chunk * chunk_tokens * k;
    const int64_t i1 = min(T, (int64_t)(chunk + 1) * chunk_tokens) * k;
    scatter_chunk(idx, cnt, off, sorted_token, row_of, i0, i1, k, E, cap, nbits);
}

// Grouped-GEMM schedule: mtile_start[g] = sum over groups g' < g of
// ceil(rows(g') / bm); group E (when n_shared) is the shared expert with T rows.
// One workgroup of 512 threads (G <= 257 groups).
__global__ __launch_bounds__(512) void schedule_kernel(const int32_t *__restrict__ offsets,
                                                       int32_t *__restrict__ mtile_start, int E,
                                                       int G, int64_t T, int bm) {
    __shared__ int s_wave[16];
    const int g = threadIdx.x;
    int tv = 0;
    if (g < G) {
        const int64_t rows = g < E ? (int64_t)(offsets[g + 1] - offsets[g]) : T;
        tv = (int)((rows + bm - 1) / bm);
    }
    int total;
    const int ts = block_exclusive_scan(tv, s_wave, total);
    if (g < G) mtile_start[g] = ts;
    if (g == 0) mtile_start[G] = total;
}

// Routing check: one thread per token row counts the rows holding an index
// outside [0, E) or one expert twice (a 256-bit set per row in registers).
__global__ __launch_bounds__(256) void check_routing_kernel(const int32_t *__restrict__ idx,
                                                            int64_t T, int k, int E,
                                                            int32_t *__restrict__ n_bad) {
    for (int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; t < T;
         t += (int64_t)gridDim.x * blockDim.x) {
        uint32_t seen[MOE_MAX_EXPERTS / 32];
#pragma unroll
        for (int q = 0; q < MOE_MAX_EXPERTS / 32; ++q) seen[q] = 0u;
        bool bad = false;
        for (int s = 0; s < k; ++s) {
            const int e = idx[t * k + s];
            if ((unsigned)e >= (unsigned)E) {
                bad = true;
                continue;
            }
            const uint32_t bit = 1u << (e & 31);
#pragma unroll
            for (int q = 0; q < MOE_MAX_EXPERTS / 32; ++q)
                if (q == (e >> 5)) {
                    bad |= (seen[q] & bit) != 0u;
                    seen[q] |= bit;
                }
        }
        if (bad) atomicAdd(n_bad, 1);
    }
}

__global__ void zero_kernel(int32_t *p) { *p = 0; }

}  // namespace

hipError_t launch_check_routing(const moe_desc &d, const int32_t *topk_idx, int32_t *n_bad,
                                hipStream_t s) {
    zero_kernel<<<1, 1, 0, s>>>(n_bad);
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(d.T, 256), 4096);
    check_routing_kernel<<<blocks, 256, 0, s>>>(topk_idx, d.T, d.k, d.E, n_bad);
    return hipGetLastError();
}

hipError_t launch_dispatch(const moe_desc &d, const Workspace &w, const int32_t *topk_idx,
                           int32_t *counts_assigned, int32_t *counts_kept, int32_t *offsets,
                           int32_t *sorted_token, int32_t *row_of, int64_t *n_dropped,
                           char *ws, hipStream_t s, int schedule_bm, bool counts_ready) {
    int32_t *chunk_counts = reinterpret_cast<int32_t *>(ws + w.chunk_counts);
    int nbits = 0;
    while ((1 << nbits) < d.E) ++nbits;
    if (!counts_ready)
        dispatch_count_kernel<<<w.n_chunks, 256, 0, s>>>(topk_idx, chunk_counts, d.T, d.k, d.E,
                                                         w.chunk_tokens);
    int32_t *mtile_start = schedule_bm > 0 ? reinterpret_cast<int32_t *>(ws + w.mtile_start) : nullptr;
    if (ceil_div(w.n_chunks, 1024 / d.E) <= kFusedPartChunks) {
        dispatch_fused_kernel<<<w.n_chunks, 1024, 0, s>>>(
            topk_idx, chunk_counts, w.n_chunks, d.E, d.T, d.k, d.capacity, counts_assigned,
            counts_kept, offsets, n_dropped, mtile_start, schedule_bm, d.n_shared, sorted_token,
            row_of, w.chunk_tokens, nbits);
        return hipGetLastError();
    }
    dispatch_scan_kernel<<<1, 1024, 0, s>>>(chunk_counts, w.n_chunks, d.E, d.T, d.k, d.capacity,
                                            counts_assigned, counts_kept, offsets, n_dropped,
                                            mtile_start, schedule_bm, d.n_shared);
    dispatch_scatter_kernel<<<w.n_chunks, 64, 0, s>>>(topk_idx, chunk_counts, offsets,
                                                      sorted_token, row_of, d.T, d.k, d.E,
                                                      d.capacity, w.chunk_tokens, nbits);
    return hipGetLastError();
}

hipError_t launch_schedule(const moe_desc &d, const int32_t *offsets, int32_t *mtile_start,
                           int bm, hipStream_t s) {
    const int G = d.E + d.n_shared;
    schedule_kernel<<<1, 512, 0, s>>>(offsets, mtile_start, d.E, G, d.T, bm);
    return hipGetLastError();
}

}  // namespace moe
