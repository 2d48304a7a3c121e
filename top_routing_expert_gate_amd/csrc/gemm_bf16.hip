// K3 (bf16): grouped expert GEMM on gfx950 matrix cores.
//
// The expert stage is the dense contraction of the layer: for each expert g
// its dispatched rows X_g (gathered from x through sorted_token) go through
//   up:   H = silu(X_g W_act^T) * (X_g W_lin^T)        (SwiGLU)
//         H = silu(X_g W_act^T + b_act)                (SiLU MLP)
//   down: Y = H W_down^T (+ b_down)
// (Expert Networks > Code Implementation, In[7]; LLMs-from-scratch MoE guide,
// "Expert forward pass"; DeepSeek 5.7, sections 1 and 4 -- the shared expert
// is one more group with every token as its rows).  Grouping rows by expert
// and running grouped GEMMs is the production form DeepSeek 5.7 names in
// section 5.
//
// Design (one kernel template for both projections):
// * tile = BM rows of one group x BN weight rows; for SwiGLU the BN weight
//   rows are BN/2 rows of W_act and the matching BN/2 rows of W_lin, so the
//   epilogue combines them in registers and only H is written;
// * a flat tile index over (M tile of any group, N tile); groups and their M
//   tiles come from a device-side prefix (mtile_start), so the grid is sized
//   from a host-known upper bound and surplus workgroups exit -- no host
//   synchronisation;
// * blockIdx -> tile is remapped so that consecutive tiles (same expert,
//   neighbouring N tiles) land on the same XCD and share its L2;
// * operands stream through LDS in 64-wide K slices, double buffered, stored
//   as 16-byte chunks with an XOR swizzle so both the row-contiguous writes
//   and the 32-row fragment reads are bank-conflict free;
// * v_mfma_f32_32x32x16_bf16 with f32 accumulators; each wave owns a
//   (BM/WM) x (BN/WN) sub-tile.
#include "moe_internal.h"

namespace moe {
namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk

enum { EPI_SWIGLU = 0, EPI_SILU_BIAS = 1, EPI_BIAS = 2 };

struct GemmParams {
    const __bf16 *A;              // x (gathered rows) or H (dispatch rows)
    const int32_t *sorted_token;  // token of each dispatch row
    const int32_t *offsets;       // [E+1] first dispatch row of each expert
    const int32_t *mtile_start;   // [G+1] first M tile of each group
    const __bf16 *W0, *W1, *bias; // routed experts: [E][N][K], [E][N][K], [E][N]
    const __bf16 *Ws0, *Ws1, *bs; // shared expert:  [N][K], [N][K], [N]
    __bf16 *C;                    // output rows: dispatch row, or shared_row0 + token
    int64_t T;
    int64_t shared_row0;
    int E, G, N, K;
};

__device__ __forceinline__ int swz(int r) { return (r & 7) ^ ((r >> 3) & 1); }

__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

template <int BM, int BN, int WM, int WN, int EPI, bool GATHER>
__global__ __launch_bounds__(WM *WN * 64) void grouped_gemm_bf16_kernel(GemmParams p) {
    constexpr int BK = 64;  // 8 chunks of 16 bytes per LDS row
    constexpr int NTH = WM * WN * 64;
    constexpr int WTM = BM / WM, WTN = BN / WN;
    constexpr int FM = WTM / 32, FN = WTN / 32;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int BNO = GATED ? BN / 2 : BN;  // output columns per tile
    constexpr int RPP = NTH / 8;              // tile rows covered per load pass
    constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    static_assert(BM % RPP == 0 && BN % RPP == 0, "tile / thread mismatch");
    static_assert(FM >= 1 && FN >= 1 && (!GATED || FN % 2 == 0), "wave tile");

    __shared__ u32x4 sA[2][BM * 8];
    __shared__ u32x4 sB[2][BN * 8];
    __shared__ int s_start[kMaxGroups + 1];

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    for (int g = tid; g <= p.G; g += NTH) s_start[g] = p.mtile_start[g];
    __syncthreads();

    // ---- tile of this workgroup (XCD-aware order) --------------------------
    const int ntn = (p.N + BNO - 1) / BNO;
    const int total = s_start[p.G] * ntn;
    const int per_xcd = (total + 7) >> 3;
    const int slot = blockIdx.x >> 3;
    if (slot >= per_xcd) return;
    const int logical = (blockIdx.x & 7) * per_xcd + slot;
    if (logical >= total) return;
    const int mt = logical / ntn;
    const int nt = logical - mt * ntn;
    int lo = 0, hi = p.G - 1;  // last group whose first tile is <= mt
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int g = lo;
    const bool shared = g >= p.E;
    const int64_t grow0 = shared ? 0 : p.offsets[g];
    const int64_t M = shared ? p.T : (int64_t)p.offsets[g + 1] - grow0;
    const int64_t m0 = (int64_t)(mt - s_start[g]) * BM;
    const int64_t crow0 = shared ? p.shared_row0 : grow0;
    const int n0 = nt * BNO;
    const int N = p.N, K = p.K;
    const int64_t wstride = (int64_t)N * K;
    const __bf16 *W0 = shared ? p.Ws0 : p.W0 + g * wstride;
    const __bf16 *W1 = GATED ? (shared ? p.Ws1 : p.W1 + g * wstride) : nullptr;
    const __bf16 *bias = EPI == EPI_SWIGLU ? nullptr
                         : shared         ? p.bs
                         : (p.bias ? p.bias + (int64_t)g * N : nullptr);

    // ---- per-thread global source rows ------------------------------------
    const int cq = tid & 7;  // 16-byte chunk within a 64-wide K slice
    const __bf16 *a_src[A_LD];
    bool a_ok[A_LD];
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = (tid >> 3) + i * RPP;
        const int64_t lr = m0 + r;
        a_ok[i] = lr < M;
        int64_t src = 0;
        if (a_ok[i]) src = GATHER ? (shared ? lr : (int64_t)p.sorted_token[grow0 + lr]) : crow0 + lr;
        a_src[i] = p.A + src * K + cq * 8;
    }
    const __bf16 *b_src[B_LD];
    bool b_ok[B_LD];
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = (tid >> 3) + i * RPP;
        int n;
        const __bf16 *Wb;
        if (GATED && r >= BN / 2) { n = n0 + r - BN / 2; Wb = W1; }
        else { n = n0 + r; Wb = W0; }
        b_ok[i] = n < N;
        b_src[i] = Wb + (int64_t)(b_ok[i] ? n : 0) * K + cq * 8;
    }

    f32x16 acc[FM][FN];
#pragma unroll
    for (int i = 0; i < FM; ++i)
#pragma unroll
        for (int j = 0; j < FN; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // rows of this wave's fragments inside the LDS tiles
    int arow[FM], brow[FN];
#pragma unroll
    for (int i = 0; i < FM; ++i) arow[i] = wm * WTM + i * 32 + (lane & 31);
#pragma unroll
    for (int j = 0; j < FN; ++j) {
        if (GATED)
            brow[j] = (j < FN / 2 ? wn * (WTN / 2) + j * 32
                                  : BN / 2 + wn * (WTN / 2) + (j - FN / 2) * 32) + (lane & 31);
        else
            brow[j] = wn * WTN + j * 32 + (lane & 31);
    }
    const int khalf = lane >> 5;

    const int KT = (K + BK - 1) / BK;
    u32x4 ra[A_LD], rb[B_LD];
    const u32x4 z4 = {0u, 0u, 0u, 0u};
    {
            const int kt_ = 0;
            const bool kok = kt_ * BK + cq * 8 < K;
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                ra[i] = (a_ok[i] && kok) ? *reinterpret_cast<const u32x4 *>(a_src[i] + kt_ * BK) : z4;
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                rb[i] = (b_ok[i] && kok) ? *reinterpret_cast<const u32x4 *>(b_src[i] + kt_ * BK) : z4;
        }
    {
            const int buf_ = 0;
#pragma unroll
            for (int i = 0; i < A_LD; ++i) {
                const int r = (tid >> 3) + i * RPP;
                sA[buf_][r * 8 + (cq ^ swz(r))] = ra[i];
            }
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const int r = (tid >> 3) + i * RPP;
                sB[buf_][r * 8 + (cq ^ swz(r))] = rb[i];
            }
        }
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) {
            const int kt_ = kt + 1;
            const bool kok = kt_ * BK + cq * 8 < K;
#pragma unroll
            for (int i = 0; i < A_LD; ++i)
                ra[i] = (a_ok[i] && kok) ? *reinterpret_cast<const u32x4 *>(a_src[i] + kt_ * BK) : z4;
#pragma unroll
            for (int i = 0; i < B_LD; ++i)
                rb[i] = (b_ok[i] && kok) ? *reinterpret_cast<const u32x4 *>(b_src[i] + kt_ * BK) : z4;
        }
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int ch = kk * 2 + khalf;
            bf16x8 af[FM], bfr[FN];
#pragma unroll
            for (int i = 0; i < FM; ++i) {
                u32x4 q = sA[buf][arow[i] * 8 + (ch ^ swz(arow[i]))];
                af[i] = __builtin_bit_cast(bf16x8, q);
            }
#pragma unroll
            for (int j = 0; j < FN; ++j) {
                u32x4 q = sB[buf][brow[j] * 8 + (ch ^ swz(brow[j]))];
                bfr[j] = __builtin_bit_cast(bf16x8, q);
            }
#pragma unroll
            for (int i = 0; i < FM; ++i)
#pragma unroll
                for (int j = 0; j < FN; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(af[i], bfr[j], acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) {
            const int buf_ = buf ^ 1;
#pragma unroll
            for (int i = 0; i < A_LD; ++i) {
                const int r = (tid >> 3) + i * RPP;
                sA[buf_][r * 8 + (cq ^ swz(r))] = ra[i];
            }
#pragma unroll
            for (int i = 0; i < B_LD; ++i) {
                const int r = (tid >> 3) + i * RPP;
                sB[buf_][r * 8 + (cq ^ swz(r))] = rb[i];
            }
        }
        __syncthreads();
    }

    // ---- epilogue ----------------------------------------------------------
    // 32x32 f32 accumulator layout: lane holds column (lane & 31) and rows
    // 8*(v/4) + 4*(lane/32) + (v%4), v = 0..15.
#pragma unroll
    for (int i = 0; i < FM; ++i) {
#pragma unroll
        for (int v = 0; v < 16; ++v) {
            const int rl = wm * WTM + i * 32 + (v >> 2) * 8 + khalf * 4 + (v & 3);
            const int64_t lr = m0 + rl;
            if (lr >= M) continue;
            __bf16 *crow = p.C + (crow0 + lr) * N;
            if (GATED) {
#pragma unroll
                for (int j = 0; j < FN / 2; ++j) {
                    const int n = n0 + wn * (WTN / 2) + j * 32 + (lane & 31);
                    if (n < N) crow[n] = (__bf16)(silu_fast(acc[i][j][v]) * acc[i][j + FN / 2][v]);
                }
            } else {
#pragma unroll
                for (int j = 0; j < FN; ++j) {
                    const int n = n0 + wn * WTN + j * 32 + (lane & 31);
                    if (n < N) {
                        float val = acc[i][j][v] + (bias ? (float)bias[n] : 0.f);
                        if (EPI == EPI_SILU_BIAS) val = silu_fast(val);
                        crow[n] = (__bf16)val;
                    }
                }
            }
        }
    }
}

template <int BM, int BN, int WM, int WN, int EPI, bool GATHER>
hipError_t launch_one(const GemmParams &p, int64_t max_mtiles, hipStream_t s) {
    constexpr int BNO = EPI == EPI_SWIGLU ? BN / 2 : BN;
    const int64_t ntn = ceil_div(p.N, BNO);
    const int64_t blocks = ceil_div(max_mtiles * ntn, 8) * 8;
    if (blocks == 0) return hipSuccess;
    grouped_gemm_bf16_kernel<BM, BN, WM, WN, EPI, GATHER>
        <<<(unsigned)blocks, WM * WN * 64, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

// Up projection (+ activation) then down projection for every group.
hipError_t launch_grouped_ffn_bf16(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                                   const ExpertArgs &a, const int32_t *mtile_start,
                                   int64_t max_mtiles, hipStream_t s) {
    static_assert(kGemmBM == 128, "tile schedule assumes BM = 128");
    const bool glu = d.expert_kind == MOE_EXPERT_SWIGLU;
    __bf16 *H = reinterpret_cast<__bf16 *>(a.ws + w.H);
    GemmParams up{};
    up.A = (const __bf16 *)a.x;
    up.sorted_token = a.sorted_token;
    up.offsets = a.offsets;
    up.mtile_start = mtile_start;
    up.W0 = (const __bf16 *)wt.w_act;
    up.W1 = (const __bf16 *)wt.w_lin;
    up.bias = (const __bf16 *)wt.b_act;
    up.Ws0 = (const __bf16 *)wt.ws_act;
    up.Ws1 = (const __bf16 *)wt.ws_lin;
    up.bs = (const __bf16 *)wt.bs_act;
    up.C = H;
    up.T = d.T;
    up.shared_row0 = w.rows_routed_max;
    up.E = d.E;
    up.G = d.E + d.n_shared;
    up.N = d.d_ff;
    up.K = d.d_model;
    hipError_t e;
    if (glu) e = launch_one<128, 256, 2, 2, EPI_SWIGLU, true>(up, max_mtiles, s);
    else e = launch_one<128, 256, 2, 2, EPI_SILU_BIAS, true>(up, max_mtiles, s);
    if (e != hipSuccess) return e;

    GemmParams dn = up;
    dn.A = H;
    dn.W0 = (const __bf16 *)wt.w_down;
    dn.W1 = nullptr;
    dn.bias = (const __bf16 *)wt.b_down;
    dn.Ws0 = (const __bf16 *)wt.ws_down;
    dn.Ws1 = nullptr;
    dn.bs = (const __bf16 *)wt.bs_down;
    dn.C = (__bf16 *)a.Y;
    dn.N = d.d_model;
    dn.K = d.d_ff;
    return launch_one<128, 256, 2, 2, EPI_BIAS, false>(dn, max_mtiles, s);
}

}  // namespace moe
