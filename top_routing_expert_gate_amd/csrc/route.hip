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
// gate_bf16: a bf16 MFMA GEMM (v_mfma_f32_16x16x32_bf16), 16-64 rows by
//            16-64 experts per block with the K dimension split over its
//            eight waves (the same split for every batch size), f32
//            accumulation, partials summed in a fixed order.  Operands are
//            loaded row-contiguous (four adjacent lanes read 64 bytes of one
//            row) and moved into the MFMA lane layout with ds_bpermute.
// gate_f32:  one thread per (token, expert) dot product in f32.
// topk:      16 or 32 lanes per token row when there are many rows, else a
//            whole wavefront (or a 2^n-lane slice of one for E <= 16); each
//            lane holds up to eight candidates as 64-bit keys (orderable
//            score << 32 | ~expert) and k rounds of an arg-max (row-local
//            DPP, or shuffles) pick the winners, lower index on ties.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

// ---------------------------------------------------------------------------
// gate, bf16 inputs, MFMA
// ---------------------------------------------------------------------------
// A block owns 16*NR token rows x 16*NT experts; its NW waves split d_model
// into NW contiguous K ranges (each a multiple of 32), accumulate with
// v_mfma_f32_16x16x32_bf16, and the partial sums are added in wave order
// through LDS.  NW is the same for every batch size, so a token's logits do
// not depend on how many other tokens share the call (batch invariance);
// only the block shape adapts to T.  Loads for two (or four) 32-wide K steps
// are issued before their MFMAs; they go through range-checked buffer
// descriptors, so rows and K slices outside the tile read as zeros without a
// select on the loaded data.
//
// The MFMA wants lane l to hold 16 bytes of row l % 16 (chunk l / 16 of the
// step), so a load in that layout has the four lanes of every quad in four
// different rows, and the texture unit spends about four times as long on it
// as on a load whose quads each read 64 contiguous bytes.  Loads are issued
// in the row-contiguous layout instead and each lane's 16 bytes are fetched
// from the lane that loaded them with four ds_bpermute (crossbar moves, no
// LDS storage): the MFMA sees the same operands, so the logits do not change.
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
// The 16 bytes lane (perm / 4) loaded, moved to this lane (four dword moves
// through the LDS crossbar, no LDS memory).
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
template <int NR, int NT, int NW>
__global__ __launch_bounds__(NW * 64) void gate_bf16_kernel(
    const __bf16 *__restrict__ x, const __bf16 *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E) {
    __shared__ float red[NW][16 * NR][16 * NT];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t row0 = (int64_t)blockIdx.x * 16 * NR;
    const int e0 = blockIdx.y * 16 * NT;
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
    int xoff[NR];  // byte offset of this lane's load row in each 16-row tile
#pragma unroll
    for (int a = 0; a < NR; ++a) {
        const int64_t row = row0 + a * 16 + lrow;
        xoff[a] = row < T ? (int)(row * d * 2) : kOOB;
    }
    int woff[NT];
#pragma unroll
    for (int j = 0; j < NT; ++j) {
        const int e = e0 + j * 16 + lrow;
        woff[j] = e < E ? e * d * 2 : kOOB;
    }
    const int kq = (((d + NW - 1) / NW) + 31) & ~31;  // K range of one wave
    const int kb = wave * kq;
    const int ke = min(d, kb + kq);
    const int kofs = 8 * lchunk;  // the 8-wide slice of a 32-wide K step this lane loads
    f32x4 acc[NR][NT];
#pragma unroll
    for (int a = 0; a < NR; ++a)
#pragma unroll
        for (int j = 0; j < NT; ++j) acc[a][j] = f32x4{0.f, 0.f, 0.f, 0.f};
    constexpr int U = NR * NT >= 8 ? 2 : 4;  // 32-wide K steps per batch of loads
    for (int k0 = kb; k0 < ke; k0 += U * 32) {
        u32x4 ar[U][NR], br[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int kk = k0 + u * 32 + kofs;
            const bool ok = kk < ke;  // d is a multiple of 8: a slice is in or out
#pragma unroll
            for (int a = 0; a < NR; ++a)
                ar[u][a] = __builtin_amdgcn_raw_buffer_load_b128(
                    rx, ok && xoff[a] != kOOB ? xoff[a] + kk * 2 : kOOB, 0, 0);
#pragma unroll
            for (int j = 0; j < NT; ++j)
                br[u][j] = __builtin_amdgcn_raw_buffer_load_b128(
                    rw, ok && woff[j] != kOOB ? woff[j] + kk * 2 : kOOB, 0, 0);
        }
        bf16x8 av[U][NR], bv[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
#pragma unroll
            for (int a = 0; a < NR; ++a) av[u][a] = to_mfma_layout(ar[u][a], perm);
#pragma unroll
            for (int j = 0; j < NT; ++j) bv[u][j] = to_mfma_layout(br[u][j], perm);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
#pragma unroll
            for (int a = 0; a < NR; ++a)
#pragma unroll
                for (int j = 0; j < NT; ++j)
                    acc[a][j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(av[u][a], bv[u][j], acc[a][j], 0, 0, 0);
    }
    // 16x16 f32 result layout: lane holds column (lane & 15), rows 4*(lane>>4) + v.
#pragma unroll
    for (int a = 0; a < NR; ++a)
#pragma unroll
        for (int j = 0; j < NT; ++j)
#pragma unroll
            for (int v = 0; v < 4; ++v)
                red[wave][a * 16 + 4 * (lane >> 4) + v][j * 16 + (lane & 15)] = acc[a][j][v];
    __syncthreads();
    for (int i = threadIdx.x; i < 16 * NR * 16 * NT; i += NW * 64) {
        const int r = i / (16 * NT), c = i % (16 * NT);
        const int64_t t = row0 + r;
        const int e = e0 + c;
        if (t >= T || e >= E) continue;
        float s = red[0][r][c];
#pragma unroll
        for (int q = 1; q < NW; ++q) s += red[q][r][c];
        logits[t * E + e] = s + (bias ? bias[e] : 0.f);
    }
}

// ---------------------------------------------------------------------------
// gate, f32 inputs
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(256) void gate_f32_kernel(
    const float *__restrict__ x, const float *__restrict__ w, const float *__restrict__ bias,
    float *__restrict__ logits, int64_t T, int d, int E) {
    const int64_t n = T * E;
    for (int64_t o = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; o < n;
         o += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = o / E;
        const int e = (int)(o - t * E);
        const float4 *xr = reinterpret_cast<const float4 *>(x + t * d);
        const float4 *wr = reinterpret_cast<const float4 *>(w + (int64_t)e * d);
        float acc = 0.f;
        for (int i = 0; i < d / 4; ++i) {
            float4 a = xr[i], b = wr[i];
            acc = fmaf(a.x, b.x, acc);
            acc = fmaf(a.y, b.y, acc);
            acc = fmaf(a.z, b.z, acc);
            acc = fmaf(a.w, b.w, acc);
        }
        logits[o] = acc + (bias ? bias[e] : 0.f);
    }
}

// ---------------------------------------------------------------------------
// top-k
// ---------------------------------------------------------------------------
__device__ __forceinline__ uint64_t make_key(float s, int e) {
    if (s == 0.0f) s = 0.0f;  // -0 ties with +0
    uint32_t u = __float_as_uint(s);
    uint32_t ord = (u & 0x80000000u) ? ~u : (u | 0x80000000u);
    return ((uint64_t)ord << 32) | (uint32_t)(~(uint32_t)e);
}

__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
    uint32_t lo = __shfl_xor((uint32_t)v, m);
    uint32_t hi = __shfl_xor((uint32_t)(v >> 32), m);
    return ((uint64_t)hi << 32) | lo;
}

// 64-bit max over the 64 lanes of a wavefront, result in every lane.  The
// first four steps stay inside 16-lane rows (DPP quad permutations and
// mirrors: plain VALU moves), the last two combine rows with row broadcasts,
// which leaves the wave maximum in lane 63; it is then read into a scalar.
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

__device__ __forceinline__ uint64_t wave_max_u64(uint64_t v) {
    v = row_max_u64(v);
    v = dpp_max_u64<0x142, 0xA>(v);  // row_bcast:15 into rows 1 and 3
    v = dpp_max_u64<0x143, 0xC>(v);  // row_bcast:31 into rows 2 and 3: lane 63 = max
    const uint32_t lo = __builtin_amdgcn_readlane((uint32_t)v, 63);
    const uint32_t hi = __builtin_amdgcn_readlane((uint32_t)(v >> 32), 63);
    return ((uint64_t)hi << 32) | lo;
}

// C = candidates per lane (experts e = sub + j*L, j < C); L = lanes per row.
// LT = 64: one row per wavefront, reductions by DPP and a scalar broadcast;
// LT = 16 or 32: four or two rows per wavefront, reductions by row-local DPP
// (plus one lane shuffle across row pairs for 32); LT = 0: L (< 16) is a
// run-time value and the reductions use lane shuffles.
// score_fn: MOE_SCORE_SOFTMAX (weights renormalised over the k selected),
// MOE_SCORE_SIGMOID, or MOE_SCORE_SOFTMAX_ALL (weights = the selected
// probabilities of the softmax over all E experts).
template <int C, int LT>
__global__ __launch_bounds__(256) void topk_kernel(
    const float *__restrict__ logits, const float *__restrict__ sel_bias,
    int32_t *__restrict__ topk_idx, float *__restrict__ topk_w, int64_t T, int E, int k,
    int score_fn, int L) {
    const bool sigmoid = score_fn == MOE_SCORE_SIGMOID;
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
        float val[C];  // logit (softmax) or affinity (sigmoid) of each candidate
        uint64_t key[C];
#pragma unroll
        for (int j = 0; j < C; ++j) {
            const int e = sub + j * L;
            const bool ok = row_ok && e < E;
            const float l = ok ? logits[row * E + e] : 0.f;
            float s = l;
            val[j] = l;
            if (sigmoid) {
                const float a = (float)(1.0 / (1.0 + exp(-(double)l)));
                val[j] = a;
                s = sel_bias ? a + sel_bias[e] : a;
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
            if (LT == 64) v = __uint_as_float(__builtin_amdgcn_readlane(__float_as_uint(v), lw));
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
                }
            }
        }
    }
}

}  // namespace

hipError_t launch_gate(const moe_desc &d, const void *x, const void *w_router,
                       const float *router_bias, float *logits, hipStream_t s) {
    if (d.dtype == MOE_BF16) {
        // enough workgroups to cover 256 CUs: wide expert tiles when T is large,
        // narrow tiles and a 16-way K split when it is small (decode)
        // the 8-way K split is the same for every T (batch-invariant logits);
        // the block shape (16 or 32 rows, 16..64 experts) adapts to T and E
        const __bf16 *xb = (const __bf16 *)x, *wb = (const __bf16 *)w_router;
        constexpr int NW = kGateWaves;
        const int nt = d.E <= 16 ? 1 : d.E <= 32 ? 2 : 4;
        const unsigned cols = (unsigned)ceil_div(d.E, 16 * nt);
        const bool two_rows = ceil_div(d.T, 32) * (int64_t)cols >= 256;
        // many experts: 64 tokens x 64 experts per workgroup when that still
        // fills the chip -- the router rows are read by half as many
        // workgroups, which outweighs reading x once more per column block
        const bool four_rows = nt == 4 && ceil_div(d.T, 64) * (int64_t)cols >= 256;
#define MOE_GATE(NR, NT)                                                                     \
    gate_bf16_kernel<NR, NT, NW><<<dim3((unsigned)ceil_div(d.T, 16 * NR), (unsigned)ceil_div(d.E, 16 * NT)), \
                                   NW * 64, 0, s>>>(xb, wb, router_bias, logits, d.T, d.d_model, d.E)
        if (four_rows) {
            MOE_GATE(4, 4);
        } else if (two_rows) {
            if (nt == 4) MOE_GATE(2, 4); else if (nt == 2) MOE_GATE(2, 2); else MOE_GATE(2, 1);
        } else if (ceil_div(d.T, 16) * (int64_t)cols >= 256) {
            if (nt == 4) MOE_GATE(1, 4); else if (nt == 2) MOE_GATE(1, 2); else MOE_GATE(1, 1);
        } else {
            MOE_GATE(1, 1);  // few tokens: narrow expert tiles for more workgroups
        }
#undef MOE_GATE
    } else {
        int64_t n = d.T * d.E;
        unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(n, 256), 65536);
        gate_f32_kernel<<<blocks, 256, 0, s>>>((const float *)x, (const float *)w_router,
                                               router_bias, logits, d.T, d.d_model, d.E);
    }
    return hipGetLastError();
}

hipError_t launch_topk(const moe_desc &d, const float *logits, const float *sel_bias,
                       int32_t *topk_idx, float *topk_w, hipStream_t s) {
    // lanes per row: a power of two >= E up to 16 experts; above that 16
    // lanes for up to 128 experts and 32 for up to 256 (several rows per
    // wavefront) when the rows still make 2048 wavefronts, else a whole
    // wavefront per row (few rows: the shorter chain per row wins); at least
    // k/4 lanes, since a lane keeps up to four of the k results
    int L = 1;
    if (d.E <= 16) {
        while (L < d.E) L <<= 1;
    } else {
        L = d.E <= 128 ? 16 : d.E <= 256 ? 32 : 64;
        if (ceil_div(d.T, 64 / L) < 2048) L = 64;
    }
    while (4 * L < d.k) L <<= 1;
    int C = 1;
    while (C * L < d.E) C <<= 1;  // candidates per lane, 1..8
    const int rows_per_block = 4 * (64 / L);
    unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(d.T, rows_per_block), 1 << 16);
    const int sig = d.score_fn;
    const float *sb = sig == MOE_SCORE_SIGMOID ? sel_bias : nullptr;
#define MOE_TOPK(CC, LL)                                                                     \
    topk_kernel<CC, LL><<<blocks, 256, 0, s>>>(logits, sb, topk_idx, topk_w, d.T, d.E, d.k, sig, L)
#define MOE_TOPK_C(LL)                                                                       \
    if (C == 1) MOE_TOPK(1, LL); else if (C == 2) MOE_TOPK(2, LL);                           \
    else if (C == 4) MOE_TOPK(4, LL); else MOE_TOPK(8, LL);
    if (L < 16) {
        MOE_TOPK(1, 0);
    } else if (L == 16) {
        MOE_TOPK_C(16)
    } else if (L == 32) {
        MOE_TOPK_C(32)
    } else {
        if (C == 1) MOE_TOPK(1, 64); else if (C == 2) MOE_TOPK(2, 64); else MOE_TOPK(4, 64);
    }
#undef MOE_TOPK_C
#undef MOE_TOPK
    return hipGetLastError();
}

}  // namespace moe
