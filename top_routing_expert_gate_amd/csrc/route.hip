// K1: gate linear layer and top-k routing for gfx950.
//
// The gate is a linear layer over each token row (MoE-router build guide,
// step 2 TopKGate; LLMs-from-scratch MoE guide, "Gate computation").  Top-k
// keeps the k best selection scores per token; weights are the softmax over
// the k selected logits (LLMs-from-scratch MoE guide, "Routing
// probabilities") or the unbiased sigmoid affinities of the selected experts
// normalised to one, the balancing bias touching the choice only (DeepSeek
// 5.7, section 2 "Score, select, then weight"), or the selected probabilities
// of the softmax over all experts left unrenormalised (MoE-router build
// guide, step 2, as its TopKGate code is written).
//
// gate_bf16: a bf16 MFMA GEMM (v_mfma_f32_16x16x32_bf16) over 16-64 token
//            rows by 16-256 experts per workgroup.  Its eight waves split
//            d_model into eight fixed K ranges, each accumulated in order,
//            and the partial sums are added in wave order: a logit's
//            arithmetic is the same for every block shape and batch size.
//            With every expert of its tokens in the block, the workgroup
//            also selects the top-k from the logits it holds in LDS (the
//            logits never go to memory unless asked for); otherwise it
//            writes the logits and topk_kernel selects.
// gate_xlds: the fused gate for 65-128 experts with d in (1792, 2048]: the
//            block's 32 rows of x are copied into LDS once and each wave
//            keeps the eight K-range sums of its 16 experts itself (the same
//            arithmetic, so the same bits as gate_bf16).
// gate_f32:  float32 layers: each lane computes whole dot products in order
//            and the same lanes then select (always fused).
// topk:      L lanes per token row (a power of two >= E up to 16 experts, 16
//            up to 128, 32 up to 256; more when k > 4L), up to eight
//            candidates per lane as 64-bit keys (orderable score << 32 |
//            ~expert), k rounds of an arg-max (row-local DPP, or shuffles),
//            lower index on ties.  The lane layout depends on E and k only,
//            so the fused and the standalone selection give the same bits.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// top-k selection of one token row held by L lanes
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t make_key(float s, int e) {
    if (s == 0.0f) s = 0.0f;  // -0 ties with +0
    uint32_t u = __float_as_uint(s);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

// The score a key was made from (-0 comes back as +0).
__device__ __forceinline__ float key_score(uint64_t key) {
    const uint32_t ord = (uint32_t)(key >> 32);
    return __uint_as_float((ord & 0x80000000u) ? (ord & 0x7FFFFFFFu) : ~ord);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// 64-bit max over lanes exchanged by one DPP pattern (plain VALU moves).
template <int CTRL, int ROW_MASK>
__device__ __forceinline__ uint64_t dpp_max_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)v, hi = (uint32_t)(v >> 32);
    const uint32_t olo = __builtin_amdgcn_update_dpp(lo, lo, CTRL, ROW_MASK, 0xF, false);
    const uint32_t ohi = __builtin_amdgcn_update_dpp(hi, hi, CTRL, ROW_MASK, 0xF, false);
    const uint64_t o = ((uint64_t)ohi << 32) | olo;
    return o > v ? o : v;
}

// 64-bit max over each 16-lane row, result in every lane of the row.
__device__ __forceinline__ uint64_t row_max_u64(uint64_t v) {
    v = dpp_max_u64<0xB1, 0xF>(v);   // quad_perm [1,0,3,2]
    v = dpp_max_u64<0x4E, 0xF>(v);   // quad_perm [2,3,0,1]
    v = dpp_max_u64<0x141, 0xF>(v);  // row_half_mirror
    v = dpp_max_u64<0x140, 0xF>(v);  // row_mirror: every lane holds its row's max
    return v;
}

// 64-bit max over the 64 lanes: row maxima, then row broadcasts leave the
// wave maximum in lane 63, read into a scalar.
__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = row_max_u64(v);
    v = dpp_max_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 = max
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// Lanes per token row and candidates per lane for E experts and top-k; the
// same for every batch size and for the fused and the standalone selection.
struct TopkLayout {
    int L, C;
};
inline TopkLayout topk_layout(int E, int k) {
    int L = 1;
    if (E <= 16) {
        while (L < E) L <<= 1;
    } else {
        L = E <= 128 ? 16 : 32;
    }
    while (4 * L < k) L <<= 1;  // a lane keeps up to four of the k results
    int C = 1;
    while (C * L < E) C <<= 1;  // 1..8
    return {L, C};
}

// Select and weigh one token row.  Lane `sub` of the row's L lanes holds the
// logits of experts e = sub + j*L in lg[j] (j < C; values for e >= E are
// ignored).  C = candidates per lane; LT = L when it is 16, 32 or 64 (the
// reductions use row-local DPP), 0 for L < 16 (shuffles; L is then the
// run-time value).  grp = the row's lane group inside the wavefront.
// score_fn: MOE_SCORE_SOFTMAX (weights renormalised over the k selected),
// MOE_SCORE_SIGMOID, or MOE_SCORE_SOFTMAX_ALL (weights = the selected
// probabilities of the softmax over all E experts).  Writes slot s = sub +
// q*L of topk_idx / topk_w (q < 4), and, when `hist` (LDS) is not NULL, adds
// one to hist[e] for every expert e it selects.  Every lane of the wavefront
// calls it.
template <int C, int LT>
__device__ __forceinline__ void route_row(const float (&lg)[C], bool row_ok, int sub, int grp,
                                          int L, int64_t row, int E, int k, int score_fn,
                                          const float *__restrict__ sel_bias,
                                          int32_t *__restrict__ topk_idx,
                                          float *__restrict__ topk_w, int *hist = nullptr) {
    const bool sigmoid = score_fn == MOE_SCORE_SIGMOID;
    float val[C];  // logit (softmax) or affinity (sigmoid) of each candidate
    uint64_t key[C];
#pragma unroll
    for (int j = 0; j < C; ++j) {
        const int e = sub + j * L;
        const bool ok = row_ok && e < E;
        const float l = ok ? lg[j] : 0.f;
        float s = l;
        val[j] = l;
        if (sigmoid) {
            const float a = (float)(1.0 / (1.0 + exp(-(double)l)));
            val[j] = a;
            s = sel_bias ? a + sel_bias[e < E ? e : 0] : a;
        }
        key[j] = ok ? make_key(s, e) : 0ull;
    }
    int my_idx[4] = {0, 0, 0, 0};
    float my_val[4] = {0.f, 0.f, 0.f, 0.f};
    for (int r = 0; r < k; ++r) {
        uint64_t best = key[0];
#pragma unroll
        for (int j = 1; j < C; ++j) best = key[j] > best ? key[j] : best;
        if (LT == 64) {
            best = wave_max_u64(best);
        } else if (LT == 16 || LT == 32) {
            best = row_max_u64(best);
            if (LT == 32) {
                const uint64_t o = shfl_xor_u64(best, 16);
                best = o > best ? o : best;
            }
        } else {
            for (int m = L >> 1; m > 0; m >>= 1) {
                uint64_t o = shfl_xor_u64(best, m);
                best = o > best ? o : best;
            }
        }
        const int ew = (int)(~(uint32_t)best);
        const int lw = ew & (L - 1);
        const int jw = ew / L;
        float v = 0.f;
#pragma unroll
        for (int j = 0; j < C; ++j) {
            if (sub == lw && j == jw) {
                v = val[j];
                key[j] = 0ull;
            }
        }
        // softmax: the winner's logit is its key's score (a -0 logit comes
        // back as +0, which weighs the same); sigmoid: its affinity, which
        // the selection offset kept out of the key, from the lane holding it
        if (!sigmoid) v = key_score(best);
        else if (LT == 64) v = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), lw));
        else v = __shfl(v, grp * L + lw);
        const int q = r / L;
        if (sub == (r & (L - 1))) {
#pragma unroll
            for (int qq = 0; qq < 4; ++qq)
                if (qq == q) {
                    my_idx[qq] = ew;
                    my_val[qq] = v;
                }
        }
    }
    // weights of this lane's slots s = sub + q*L
    float contrib[4];
    float part = 0.f;
    const float m0 = __shfl(my_val[0], grp * L);  // slot 0 holds the largest logit
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const bool has = sub + q * L < k;
        float c = 0.f;
        if (has) c = sigmoid ? my_val[q] : expf(my_val[q] - m0);
        contrib[q] = c;
        part += c;
    }
    if (score_fn == MOE_SCORE_SOFTMAX_ALL) {
        // denominator over every expert of the row; m0 is the row maximum
        part = 0.f;
#pragma unroll
        for (int j = 0; j < C; ++j)
            if (sub + j * L < E) part += expf(val[j] - m0);
    }
    for (int m = L >> 1; m > 0; m >>= 1) part += __shfl_xor(part, m);
    if (row_ok) {
#pragma unroll
        for (int q = 0; q < 4; ++q) {
            const int s = sub + q * L;
            if (s < k) {
                topk_idx[row * k + s] = my_idx[q];
                topk_w[row * k + s] = contrib[q] / part;
                if (hist) atomicAdd(&hist[my_idx[q]], 1);
            }
        }
    }
}

// ---------------------------------------------------------------------------
// gate, bf16 inputs, MFMA (optionally with the selection fused)
// ---------------------------------------------------------------------------
// A block owns 16*NR token rows x 16*NT experts; its 8 waves split d_model
// into 8 contiguous K ranges (each a multiple of 32), accumulate with
// v_mfma_f32_16x16x32_bf16 in K order, and the partial sums are added in wave
// order through LDS.  The split is the same for every batch size and block
// shape, so a token's logits do not depend on how many other tokens share the
// call or which kernel shape computes them.
//
// Loads run DEPTH 32-wide K steps ahead of the products through a ring of
// register sets: the gate moves few bytes per CU and is bound by the latency
// of its loads, so as many as the registers allow are kept in flight.  They
// go through range-checked buffer descriptors: rows and K slices outside the
// tile read as zeros without a select on the loaded data.
//
// The MFMA wants lane l to hold 16 bytes of row l % 16 (chunk l / 16 of the
// step), so a load in that layout has the four lanes of every quad in four
// different rows, and the texture unit spends about four times as long on it
// as on a load whose quads each read 64 contiguous bytes.  Loads are issued
// in the row-contiguous layout instead and each lane's 16 bytes are fetched
// from the lane that loaded them with four ds_bpermute (crossbar moves, no
// LDS storage): the MFMA sees the same operands.
__device__ __forceinline__ bf16x8 to_mfma_layout(u32x4 v, int perm) {
    u32x4 r;
    r.x = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)v.x);
    r.y = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)v.y);
    r.z = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)v.z);
    r.w = (uint32_t)__builtin_amdgcn_ds_bpermute(perm, (int)v.w);
    return __builtin_bit_cast(bf16x8, r);
}
constexpr int kGateWaves = 8;
constexpr int kRsrcWord3 = 0x00020000;  // gfx9-family raw buffer descriptor word
constexpr int kOOB = (int)0x80000000u;  // an offset beyond every resource

template <int NR, int NT>
struct GateSmem {
    static constexpr int kBytes = kGateWaves * 16 * NR * 16 * NT * 4;
};

// TOPK: the block holds every expert (16*NT >= E) and selects; logits go to
// `logits` only when it is not NULL.  Otherwise the logits are written and
// C, LT are unused.
template <int NR, int NT, int DEPTH, bool TOPK, int C, int LT>
__global__ __launch_bounds__(kGateWaves * 64) void gate_bf16_kernel(
    const __bf16 *__restrict__ x, const __bf16 *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E, int k, int score_fn,
    const float *__restrict__ sel_bias, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int L, int32_t *__restrict__ chunk_counts) {
    constexpr int NW = kGateWaves;
    constexpr int NL = NR + NT;  // 16-byte loads per lane per K step
    __shared__ float red[NW][16 * NR][16 * NT];
    // fused selection with chunk_counts: the block's expert histogram (the
    // dispatch's per-chunk counts, the block's rows being one chunk)
    __shared__ int hist[TOPK ? MOE_MAX_EXPERTS : 1];
    if (TOPK && chunk_counts)
        for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    const int lane = threadIdx.x & 63;
    // wave-uniform: the K range and step count below are scalar, so the load
    // ring's step test is a scalar branch and its loads stay in flight
    // across the loop (a per-lane test ends every round with a full wait)
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = (int64_t)blockIdx.x * 16 * NR;
    const int e0 = TOPK ? 0 : blockIdx.y * 16 * NT;
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(x), (short)0, (int)(T * d * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(w), (short)0, (int)((int64_t)E * d * 2), kRsrcWord3);
    // Loads are row-contiguous: lane l reads row (l >> 2) & 15 of a 16-row
    // tile, 16-byte chunk l & 3 of a 32-wide k step, so four adjacent lanes
    // read 64 contiguous bytes of one row.  The MFMA wants lane l to hold row
    // l & 15, chunk l >> 4: four ds_bpermute moves per fragment take each
    // lane's 16 bytes from lane 4 * (l & 15) + (l >> 4).
    const int lrow = (lane >> 2) & 15, lchunk = lane & 3;
    const int perm = (4 * (lane & 15) + (lane >> 4)) * 4;  // ds_bpermute byte address
    int off[NL];  // byte offset of this lane's load row: NR token tiles, then NT expert tiles
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        const int64_t row = row0 + a * 16 + lrow;
        off[a] = row < T ? (int)(row * d * 2) : kOOB;
    }
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int e = e0 + j * 16 + lrow;
        off[NR + j] = e < E ? e * d * 2 : kOOB;
    }
    const int kq = (((d + NW - 1) / NW) + 31) & ~31;  // K range of one wave
    const int kb = wave * kq;
    const int ke = min(d, kb + kq);
    const int nsteps = ke > kb ? (ke - kb + 31) / 32 : 0;
    const int kofs = 8 * lchunk;  // the 8-wide slice of a 32-wide K step this lane loads
    f32x4 acc[NR][NT];
#pragma unroll
    for (int a = 0; a < NR; ++a)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[a][j] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ring of DEPTH register sets; set u holds K steps u, u + DEPTH, ...
    u32x4 ring[DEPTH][NL];
    auto issue = [&](int step, u32x4(&dst)[NL]) {
        const int kk = kb + step * 32 + kofs;
        const bool ok = kk < ke;  // d is a multiple of 8: a slice is in or out
#pragma unroll
        for (int a = 0; a < NR; ++a)
            dst[a] = __builtin_amdgcn_raw_buffer_load_b128(
                rx, ok && off[a] != kOOB ? off[a] + kk * 2 : kOOB, 0, 0);
#pragma unroll
        for (int j = 0; j < NT; ++j)
            dst[NR + j] = __builtin_amdgcn_raw_buffer_load_b128(
                rw, ok && off[NR + j] != kOOB ? off[NR + j] + kk * 2 : kOOB, 0, 0);
    };
    auto consume = [&](const u32x4(&src)[NL]) {
        bf16x8 av[NR];
#pragma unroll
        for (int a = 0; a < NR; ++a) av[a] = to_mfma_layout(src[a], perm);
#pragma unroll
        for (int j = 0; j < NT; ++j) {
            const bf16x8 bv = to_mfma_layout(src[NR + j], perm);
#pragma unroll
            for (int a = 0; a < NR; ++a)
                acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[a], bv, acc[a][j], 0, 0, 0);
        }
    };
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) issue(u, ring[u]);
    // whole rounds of DEPTH steps with no test inside, so that the wait for a
    // step's loads leaves the DEPTH-1 newer sets in flight; the last round's
    // requests past the K range read zeros and fetch nothing
    int i = 0;
    for (; i + DEPTH <= nsteps; i += DEPTH) {
#pragma unroll
        for (int u = 0; u < DEPTH; ++u) {
            consume(ring[u]);
            issue(i + u + DEPTH, ring[u]);
        }
    }
#pragma unroll
    for (int u = 0; u < DEPTH - 1; ++u)
        if (i + u < nsteps) consume(ring[u]);
    // 16x16 f32 result layout: lane holds column (lane & 15), rows 4*(lane>>4) + v.
#pragma unroll
    for (int a = 0; a < NR; ++a)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][a * 16 + 4 * (lane >> 4) + v][j * 16 + (lane & 15)] = acc[a][j][v];
    __syncthreads();
    // logits = partials summed in wave order, plus the router offset
    for (int i = threadIdx.x; i < 16 * NR * 16 * NT; i += NW * 64) {
        const int r = i / (16 * NT), c = i % (16 * NT);
        const int64_t t = row0 + r;
        const int e = e0 + c;
        float s = red[0][r][c];
#pragma unroll
        for (int q = 1; q < NW; ++q) s += red[q][r][c];
        s = s + (bias && e < E ? bias[e] : 0.f);
        if (TOPK) red[0][r][c] = s;
        if (t < T && e < E && logits) logits[t * E + e] = s;
    }
    if (TOPK) {
        __syncthreads();
        const int Lr = LT ? LT : L;
        const int sub = lane & (Lr - 1);
        const int grp = lane / Lr;
        const int rpw = 64 / Lr;  // rows per wavefront pass
        for (int rb = wave * rpw; rb < 16 * NR; rb += NW * rpw) {
            const int r = rb + grp;
            const bool ok = r < 16 * NR && row0 + r < T;
            float lg[C];
#pragma unroll
            for (int j = 0; j < C; ++j) {
                const int e = sub + j * Lr;
                lg[j] = ok && e < 16 * NT ? red[0][r][e] : 0.f;
            }
            route_row<C, LT>(lg, ok, sub, grp, Lr, row0 + r, E, k, score_fn, sel_bias, topk_idx,
                             topk_w, chunk_counts ? hist : nullptr);
        }
        if (chunk_counts) {
            __syncthreads();
            for (int e = threadIdx.x; e < E; e += blockDim.x)
                chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
        }
    }
}

// ---------------------------------------------------------------------------
// gate + selection, bf16, 32 tokens x up to 128 experts, x held in LDS
// ---------------------------------------------------------------------------
// The block's 32 rows of x (d <= 2048) are copied into LDS once, straight
// from memory (buffer_load ... lds), and wave w owns experts 16w..16w+15 for
// all of d.  It keeps one accumulator per K range -- the same eight ranges,
// each a chain of v_mfma_f32_16x16x32_bf16 in K order, as gate_bf16_kernel's
// waves -- and adds the eight in range order at the end, so each logit is
// the same bits as there, with no partial sums passed between waves.  The
// router rows stream through a register ring (row-contiguous loads moved
// into the MFMA layout with ds_bpermute); the x fragments are read from LDS.
// Row t of x sits at t * P 16-byte chunks, chunk c at position c ^ (t & 15),
// so the 16 rows of a fragment read fall in 16 different bank groups.
constexpr int kXldsRows = 32;
constexpr int kXldsMaxChunks = 256;  // 16-byte chunks per row: d <= 2048

template <int C, int LT>
__global__ __launch_bounds__(kGateWaves * 64) void gate_xlds_kernel(
    const __bf16 *__restrict__ x, const __bf16 *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E, int k, int score_fn,
    const float *__restrict__ sel_bias, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int L, int32_t *__restrict__ chunk_counts) {
    // eight router steps in flight per wave: measured against 4, 6, 12, 16,
    // 24 and 32 at the headline shape, 8 was fastest (21.2 us per call with x
    // in cache and 30.7 us from HBM, against 22.0 / 31.5 us with 16); deeper
    // rings put more requests ahead of the first quarter of x
    constexpr int NW = kGateWaves, DEPTH = 8, AHEAD = 2;
    // x rows in four K quarters of 512 (64 chunks of every row each); after
    // the K loop the first holds the block's logits [32][128]
    __shared__ __attribute__((aligned(16))) u32x4 xq0[kXldsRows * 64];
    __shared__ __attribute__((aligned(16))) u32x4 xq1[kXldsRows * 64];
    __shared__ __attribute__((aligned(16))) u32x4 xq2[kXldsRows * 64];
    __shared__ __attribute__((aligned(16))) u32x4 xq3[kXldsRows * 64];
    __shared__ int hist[MOE_MAX_EXPERTS];
    float(*lg_s)[128] = reinterpret_cast<float(*)[128]>(xq0);
    if (chunk_counts)
        for (int e = threadIdx.x; e < E; e += blockDim.x) hist[e] = 0;
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t row0 = (int64_t)blockIdx.x * kXldsRows;
    const int cpr = d >> 3;                  // 16-byte chunks per row of x (225..256)
    const __amdgpu_buffer_rsrc_t rx = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(x), (short)0, (int)(T * d * 2), kRsrcWord3);
    const __amdgpu_buffer_rsrc_t rw = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<__bf16 *>(w), (short)0, (int)((int64_t)E * d * 2), kRsrcWord3);

    // ---- router ring: lane l loads expert row (l >> 2) & 15 of this wave's
    // 16, chunk l & 3 of a 32-wide k step; four ds_bpermute put it in the
    // MFMA layout (lane l: row l & 15, chunk l >> 4)
    const int lrow = (lane >> 2) & 15, lchunk = lane & 3;
    const int perm = (4 * (lane & 15) + (lane >> 4)) * 4;
    const int e_load = wave * 16 + lrow;
    const int woff = e_load < E ? e_load * d * 2 : kOOB;
    u32x4 ring[DEPTH];
    auto issue = [&](int step, u32x4 &dst) {
        const int kk = step * 32 + 8 * lchunk;
        dst = __builtin_amdgcn_raw_buffer_load_b128(
            rw, kk < d && woff != kOOB ? woff + kk * 2 : kOOB, 0, 0);
    };
    // ---- quarter q of x into LDS: this wave requests rows wave + 8i (i < 4);
    // a request covers the row's 64 chunks of the quarter, chunk c landing at
    // position (c - 64q) ^ (row & 15); chunks at or past d read as zeros
    auto x_quarter = [&](int q, u32x4 *dst) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tr = wave + 8 * i;
            const int c = 64 * q + (lane ^ (tr & 15));
            const int64_t row = row0 + tr;
            const int off = row < T && c < cpr ? (int)(row * d * 2) + c * 16 : kOOB;
            __builtin_amdgcn_raw_ptr_buffer_load_lds(
                rx, (__attribute__((address_space(3))) void *)(dst + tr * 64), 16, off, 0, 0, 0);
        }
    };
#pragma unroll
    for (int u = 0; u < DEPTH; ++u) issue(u, ring[u]);
    x_quarter(0, xq0);
    x_quarter(1, xq1);
    x_quarter(2, xq2);
    x_quarter(3, xq3);
    // a plain barrier, not __syncthreads: its release fence would also wait
    // for quarters 1-3, which stay in flight
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0x0F7C);  // vmcnt(12): the ring's first loads and quarter 0 landed
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");

    // ---- K loop: 64 steps of 32 over d in (1792, 2048], in eight ranges of
    // eight steps (kq = 256, as in gate_bf16_kernel), unrolled so that the
    // range, the ring slot and the LDS quarter of every step are known at
    // compile time.  Step g's router fragment comes from slot g % DEPTH,
    // which is then refilled with step g + DEPTH; its operands are gathered
    // AHEAD steps early so that the crossbar and LDS latency overlap the
    // products before.  All four quarters of x are requested at the start;
    // the loop starts once quarter 0 has landed, and the rest is waited for
    // (then all waves meet) before step 16 is gathered: the 16 ring refills
    // issued after the quarters are all that may still be in flight then
    // (waiting for a refill waits for every request issued before it, so
    // quarters 1-3 cannot be left for later; with eight sets the wait for
    // step 8's refill already covers them).  Steps past d multiply
    // zeros (both operands are zero there), which leaves the sums as they
    // are: the same bits as a range that stops at d.  Waves whose experts
    // all lie past E multiply zeros too (their logits are not kept).
    f32x4 acc[NW][2];
#pragma unroll
    for (int r = 0; r < NW; ++r) acc[r][0] = acc[r][1] = f32x4{0.f, 0.f, 0.f, 0.f};
    const int fr = lane & 15, fc = lane >> 4;  // fragment row / chunk of this lane
    bf16x8 bq[AHEAD + 1];
    u32x4 xv[AHEAD + 1][2];
    auto gather = [&](int g) {  // operands of step g into set g % (AHEAD + 1)
        u32x4 &slot = ring[g % DEPTH];
        bq[g % (AHEAD + 1)] = to_mfma_layout(slot, perm);
        issue(g + DEPTH, slot);
        const u32x4 *xqs = g < 16 ? xq0 : g < 32 ? xq1 : g < 48 ? xq2 : xq3;
        const int c = (4 * g + fc) & 63;
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) xv[g % (AHEAD + 1)][tt] = xqs[(16 * tt + fr) * 64 + (c ^ fr)];
    };
#pragma unroll
    for (int g = 0; g < AHEAD; ++g) gather(g);
#pragma unroll
    for (int g = 0; g < 64; ++g) {
        const int gn = g + AHEAD;  // the step gathered now
        if (gn == 16) {
            __builtin_amdgcn_sched_barrier(0);
            __builtin_amdgcn_s_waitcnt(0x4F70);  // vmcnt(16) (high bits 15:14 = 1)
            __builtin_amdgcn_s_barrier();
            asm volatile("" ::: "memory");
            __builtin_amdgcn_sched_barrier(0);
        }
        if (gn < 64) gather(gn);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
            acc[g / 8][tt] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(
                __builtin_bit_cast(bf16x8, xv[g % (AHEAD + 1)][tt]), bq[g % (AHEAD + 1)],
                acc[g / 8][tt], 0, 0, 0);
    }
    const bool active = wave * 16 < E;        // wave-uniform
    __builtin_amdgcn_s_waitcnt(0x0070);  // drain the ring's look-ahead past d
    __syncthreads();                     // every wave is done with x in LDS

    // ---- logits = the eight range sums in range order, plus the router offset
    if (active) {
        const int e = wave * 16 + (lane & 15);
#pragma unroll
        for (int tt = 0; tt < 2; ++tt)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int tl = 16 * tt + 4 * (lane >> 4) + v;
                float s = acc[0][tt][v];
#pragma unroll
                for (int r = 1; r < NW; ++r) s += acc[r][tt][v];
                s = s + (bias && e < E ? bias[e] : 0.f);
                lg_s[tl][e] = s;
                const int64_t t = row0 + tl;
                if (t < T && e < E && logits) logits[t * E + e] = s;
            }
    }
    __syncthreads();
    // ---- selection of the block's 32 rows
    const int Lr = LT ? LT : L;
    const int sub = lane & (Lr - 1);
    const int grp = lane / Lr;
    const int rpw = 64 / Lr;
    for (int rb = wave * rpw; rb < kXldsRows; rb += NW * rpw) {
        const int r = rb + grp;
        const bool ok = r < kXldsRows && row0 + r < T;
        float lg[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int e = sub + j * Lr;
            lg[j] = ok && e < E ? lg_s[r][e] : 0.f;
        }
        route_row<C, LT>(lg, ok, sub, grp, Lr, row0 + r, E, k, score_fn, sel_bias, topk_idx,
                         topk_w, chunk_counts ? hist : nullptr);
    }
    if (chunk_counts) {
        __syncthreads();
        for (int e = threadIdx.x; e < E; e += blockDim.x)
            chunk_counts[(int64_t)blockIdx.x * E + e] = hist[e];
    }
}

// ---------------------------------------------------------------------------
// gate + selection, f32 inputs
// ---------------------------------------------------------------------------
// L lanes per token row; lane `sub` computes the dot products of experts
// sub + j*L in d order (one fused multiply-add per element), adds the router
// offset, and the row's lanes select.
template <int C, int LT>
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E, int k, int score_fn,
    const float *__restrict__ sel_bias, int32_t *__restrict__ topk_idx,
    float *__restrict__ topk_w, int L) {
    if (LT) L = LT;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (L - 1);
    const int grp = lane / L;
    const int R = 64 / L;  // rows per wavefront
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t base = gw * R; base < T; base += nw * R) {
        const int64_t row = base + grp;
        const bool row_ok = row < T;
        float lg[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int e = sub + j * L;
            float acc = 0.f;
            if (row_ok && e < E) {
                const float4 *xr = reinterpret_cast<const float4 *>(x + row * d);
                const float4 *wr = reinterpret_cast<const float4 *>(w + (int64_t)e * d);
                for (int i = 0; i < d / 4; ++i) {
                    const float4 a = xr[i], b = wr[i];
                    acc = fmaf(a.x, b.x, acc);
                    acc = fmaf(a.y, b.y, acc);
                    acc = fmaf(a.z, b.z, acc);
                    acc = fmaf(a.w, b.w, acc);
                }
                acc = acc + (bias ? bias[e] : 0.f);
                if (logits) logits[row * E + e] = acc;
            }
            lg[j] = acc;
        }
        route_row<C, LT>(lg, row_ok, sub, grp, L, row, E, k, score_fn, sel_bias, topk_idx, topk_w);
    }
}

// ---------------------------------------------------------------------------
// top-k from logits in memory
// ---------------------------------------------------------------------------
template <int C, int LT>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ logits, const float *__restrict__ sel_bias,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int64_t T, int E, int k,
    int score_fn, int L) {
    if (LT) L = LT;
    const int lane = threadIdx.x & 63;
    const int sub = lane & (L - 1);
    const int grp = lane / L;
    const int R = 64 / L;  // rows per wavefront
    const int64_t gw = (int64_t)blockIdx.x * (blockDim.x >> 6) + (threadIdx.x >> 6);
    const int64_t nw = (int64_t)gridDim.x * (blockDim.x >> 6);
    for (int64_t base = gw * R; base < T; base += nw * R) {
        const int64_t row = base + grp;
        const bool row_ok = row < T;
        float lg[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int e = sub + j * L;
            lg[j] = row_ok && e < E ? logits[row * E + e] : 0.f;
        }
        route_row<C, LT>(lg, row_ok, sub, grp, L, row, E, k, score_fn, sel_bias, topk_idx, topk_w);
    }
}

// ---------------------------------------------------------------------------
// launchers
// ---------------------------------------------------------------------------
struct RouteArgs {
    const moe_desc *d;
    const void *x;
    const void *w_router;
    const float *router_bias;
    const float *sel_bias;  // already NULL unless sigmoid routing
    float *logits;          // NULL: not written (fused paths only)
    int32_t *topk_idx;
    float *topk_w;
    int32_t *chunk_counts;  // fused bf16 path: per-block expert counts, or NULL
};

unsigned rows_blocks(int64_t T, int rows_per_block) {
    return (unsigned)std::min<int64_t>(ceil_div(T, rows_per_block), 1 << 16);
}

// f32: always fused
hipError_t launch_route_f32(const RouteArgs &a, hipStream_t s) {
    const moe_desc &d = *a.d;
    const TopkLayout lay = topk_layout(d.E, d.k);
    const unsigned blocks = rows_blocks(d.T, 4 * (64 / lay.L));
#define MOE_GF(CC, LL)                                                                       \
    gate_f32_kernel<CC, LL><<<blocks, 256, 0, s>>>(                                          \
        (const float *)a.x, (const float *)a.w_router, a.router_bias, a.logits, d.T, d.d_model, \
        d.E, d.k, d.score_fn, a.sel_bias, a.topk_idx, a.topk_w, lay.L)
#define MOE_GF_C(LL)                                                                         \
    if (lay.C == 1) MOE_GF(1, LL); else if (lay.C == 2) MOE_GF(2, LL);                      \
    else if (lay.C == 4) MOE_GF(4, LL); else MOE_GF(8, LL);
    if (lay.L < 16) {
        MOE_GF(1, 0);
    } else if (lay.L == 16) {
        MOE_GF_C(16)
    } else if (lay.L == 32) {
        MOE_GF_C(32)
    } else {
        if (lay.C == 1) MOE_GF(1, 64); else if (lay.C == 2) MOE_GF(2, 64); else MOE_GF(4, 64);
    }
#undef MOE_GF_C
#undef MOE_GF
    return hipGetLastError();
}

// bf16, fused: blocks of 16*NR tokens x every expert
template <int NR, int NT, int DEPTH>
hipError_t launch_gate_fused(const RouteArgs &a, hipStream_t s) {
    const moe_desc &d = *a.d;
    const TopkLayout lay = topk_layout(d.E, d.k);
    const dim3 grid((unsigned)ceil_div(d.T, 16 * NR), 1);
#define MOE_GB(CC, LL)                                                                       \
    gate_bf16_kernel<NR, NT, DEPTH, true, CC, LL><<<grid, kGateWaves * 64, 0, s>>>(          \
        (const __bf16 *)a.x, (const __bf16 *)a.w_router, a.router_bias, a.logits, d.T,        \
        d.d_model, d.E, d.k, d.score_fn, a.sel_bias, a.topk_idx, a.topk_w, lay.L,            \
        a.chunk_counts)
    // layouts that topk_layout can produce for 16*(NT/2) < E <= 16*NT
    if constexpr (NT == 1) {
        if (lay.L < 16) MOE_GB(1, 0); else MOE_GB(1, 16);
    } else if constexpr (NT == 2) {
        MOE_GB(2, 16);
    } else if constexpr (NT == 4) {
        MOE_GB(4, 16);
    } else if constexpr (NT == 8) {
        if (lay.L == 16) MOE_GB(8, 16); else MOE_GB(4, 32);
    } else {
        if (lay.L == 32) MOE_GB(8, 32); else MOE_GB(4, 64);
    }
#undef MOE_GB
    return hipGetLastError();
}

// bf16, logits only: blocks of 16*NR tokens x 16*NT experts
template <int NR, int NT, int DEPTH>
hipError_t launch_gate_split(const RouteArgs &a, hipStream_t s) {
    const moe_desc &d = *a.d;
    const dim3 grid((unsigned)ceil_div(d.T, 16 * NR), (unsigned)ceil_div(d.E, 16 * NT));
    gate_bf16_kernel<NR, NT, DEPTH, false, 1, 0><<<grid, kGateWaves * 64, 0, s>>>(
        (const __bf16 *)a.x, (const __bf16 *)a.w_router, a.router_bias, a.logits, d.T, d.d_model,
        d.E, d.k, d.score_fn, nullptr, nullptr, nullptr, 1, nullptr);
    return hipGetLastError();
}

// The fused gate's shape: 16*NT experts per block (every expert of the
// layer) and 16*NR tokens, NR chosen so that the partial sums fit in LDS.
// The one table for the launch and for the dispatch chunk it counts.
constexpr int fused_nt(int E) { return E <= 16 ? 1 : E <= 32 ? 2 : E <= 64 ? 4 : E <= 128 ? 8 : 16; }
constexpr int fused_nr(int nt) { return nt <= 2 ? 4 : nt <= 8 ? 2 : 1; }

// The x-in-LDS gate for 65..128 experts: x's 32 rows must fit in LDS
// (d <= 2048) and the eight K ranges must be 256 wide (d > 1792), which its
// unrolled step loop assumes.
bool xlds_gate_fits(const moe_desc &d) {
    if (fused_nt(d.E) != 8 || d.d_model > 8 * kXldsMaxChunks || d.d_model % 8 != 0) return false;
    const int kq = (((d.d_model + kGateWaves - 1) / kGateWaves) + 31) & ~31;
    return kq == 256;
}

hipError_t launch_gate_xlds(const RouteArgs &a, hipStream_t s) {
    const moe_desc &d = *a.d;
    const TopkLayout lay = topk_layout(d.E, d.k);
    const dim3 grid((unsigned)ceil_div(d.T, kXldsRows), 1);
#define MOE_GX(CC, LL)                                                                       \
    gate_xlds_kernel<CC, LL><<<grid, kGateWaves * 64, 0, s>>>(                               \
        (const __bf16 *)a.x, (const __bf16 *)a.w_router, a.router_bias, a.logits, d.T,        \
        d.d_model, d.E, d.k, d.score_fn, a.sel_bias, a.topk_idx, a.topk_w, lay.L,            \
        a.chunk_counts)
    if (lay.L == 16) MOE_GX(8, 16); else MOE_GX(4, 32);
#undef MOE_GX
    return hipGetLastError();
}

hipError_t launch_fused_bf16(const RouteArgs &a, hipStream_t s) {
    if (xlds_gate_fits(*a.d)) return launch_gate_xlds(a, s);
    switch (fused_nt(a.d->E)) {
        case 1: return launch_gate_fused<fused_nr(1), 1, 8>(a, s);
        case 2: return launch_gate_fused<fused_nr(2), 2, 4>(a, s);
        case 4: return launch_gate_fused<fused_nr(4), 4, 4>(a, s);
        case 8: return launch_gate_fused<fused_nr(8), 8, 3>(a, s);
        default: return launch_gate_fused<fused_nr(16), 16, 2>(a, s);
    }
}

hipError_t launch_split_bf16(const RouteArgs &a, hipStream_t s) {
    // enough workgroups to cover 256 CUs: wide expert tiles when T is large,
    // narrow ones when it is small (decode)
    const moe_desc &d = *a.d;
    const int nt = d.E <= 16 ? 1 : d.E <= 32 ? 2 : 4;
    const int64_t cols = ceil_div(d.E, 16 * nt);
    if (nt == 4 && ceil_div(d.T, 64) * cols >= 256) return launch_gate_split<4, 4, 4>(a, s);
    if (ceil_div(d.T, 32) * cols >= 256) {
        if (nt == 4) return launch_gate_split<2, 4, 4>(a, s);
        if (nt == 2) return launch_gate_split<2, 2, 6>(a, s);
        return launch_gate_split<2, 1, 8>(a, s);
    }
    if (ceil_div(d.T, 16) * cols >= 256) {
        if (nt == 4) return launch_gate_split<1, 4, 6>(a, s);
        if (nt == 2) return launch_gate_split<1, 2, 8>(a, s);
    }
    return launch_gate_split<1, 1, 8>(a, s);  // few tokens: narrow tiles, more workgroups
}

}  // namespace

hipError_t launch_topk(const moe_desc &d, const float *logits, const float *sel_bias,
                       int32_t *topk_idx, float *topk_w, hipStream_t s) {
    const TopkLayout lay = topk_layout(d.E, d.k);
    const unsigned blocks = rows_blocks(d.T, 4 * (64 / lay.L));
    const int sig = d.score_fn;
    const float *sb = sig == MOE_SCORE_SIGMOID ? sel_bias : nullptr;
#define MOE_TOPK(CC, LL)                                                                     \
    topk_kernel<CC, LL><<<blocks, 256, 0, s>>>(logits, sb, topk_idx, topk_w, d.T, d.E, d.k, sig, lay.L)
#define MOE_TOPK_C(LL)                                                                       \
    if (lay.C == 1) MOE_TOPK(1, LL); else if (lay.C == 2) MOE_TOPK(2, LL);                  \
    else if (lay.C == 4) MOE_TOPK(4, LL); else MOE_TOPK(8, LL);
    if (lay.L < 16) {
        MOE_TOPK(1, 0);
    } else if (lay.L == 16) {
        MOE_TOPK_C(16)
    } else if (lay.L == 32) {
        MOE_TOPK_C(32)
    } else {
        if (lay.C == 1) MOE_TOPK(1, 64); else if (lay.C == 2) MOE_TOPK(2, 64); else MOE_TOPK(4, 64);
    }
#undef MOE_TOPK_C
#undef MOE_TOPK
    return hipGetLastError();
}

int route_block_rows(const moe_desc &d) { return 16 * fused_nr(fused_nt(d.E)); }

bool route_fused_faster(const moe_desc &d) {
    if (d.dtype != MOE_BF16) return true;
    // the fused gate streams the whole router through every workgroup; keep
    // it where that is small and the token blocks still cover the chip
    return (int64_t)d.E * d.d_model * 2 <= (1 << 20) && ceil_div(d.T, route_block_rows(d)) >= 128;
}

int route_chunk_tokens(const moe_desc &d) {
    if (d.dtype != MOE_BF16 || !route_fused_faster(d)) return 0;
    return route_block_rows(d);
}

hipError_t launch_route(const moe_desc &d, const void *x, const void *w_router,
                        const float *router_bias, const float *sel_bias, float *logits,
                        float *logits_buf, int32_t *topk_idx, float *topk_w, hipStream_t s,
                        int32_t *chunk_counts) {
    RouteArgs a{&d, x, w_router, router_bias,
                d.score_fn == MOE_SCORE_SIGMOID ? sel_bias : nullptr, logits, topk_idx, topk_w,
                nullptr};
    if (d.dtype != MOE_BF16) return launch_route_f32(a, s);
    float *buf = logits ? logits : logits_buf;
    if (buf == nullptr || route_fused_faster(d)) {
        if (route_chunk_tokens(d) > 0) a.chunk_counts = chunk_counts;
        return launch_fused_bf16(a, s);
    }
    a.logits = buf;
    hipError_t e = launch_split_bf16(a, s);
    if (e != hipSuccess) return e;
    return launch_topk(d, buf, sel_bias, topk_idx, topk_w, s);
}

}  // namespace moe
