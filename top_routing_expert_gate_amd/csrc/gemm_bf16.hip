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
// Two kernels, each instantiated for both projections:
// * grouped_gemm_r5_kernel (many rows per expert: prefill and larger batches).
//   256 activation rows x 256 weight rows per tile, 8 waves of 128 x 64; for
//   SwiGLU the 256 weight rows are 128 rows of W_act and the matching 128 of
//   W_lin, so H = silu(a) * b is formed in registers and only H is written.
//   Operands go from global memory straight into LDS (buffer_load ... lds) in
//   64-wide K slices, eight lanes per 128-byte row segment; each slice's
//   activation and weight halves rotate through five 32 KiB slots, weights
//   requested two slices ahead, activations one.  Fragment reads of the next
//   16-wide k step are issued between the products of the current one, and
//   the last step's products run after the barrier that ends the slice.
// * grouped_gemm_bf16_kernel<32, 256, 1, 4> (a handful of rows per expert:
//   decode): register-staged double-buffered 64-wide K slices; bound by
//   streaming each touched expert's weights once.
// Common to both:
// * a flat tile index over (M tile of any group, N tile); the groups' M-tile
//   prefix (mtile_start) is built on the device, the grid is sized from a
//   host-known upper bound and surplus workgroups exit: no host sync.
// * blockIdx -> tile is remapped so that consecutive tiles run on one XCD and
//   share its L2; the five-slot kernel also orders a group's tiles in bands
//   of 8 M tiles (N tiles of a band one after another, each over the band's
//   M tiles), so the readers of a weight panel start close together.
// * 16-byte LDS chunks XOR-swizzled so that the 32-row fragment reads are
//   bank-conflict free.
// * v_mfma_f32_32x32x16_bf16 with the WEIGHT fragment as the first operand:
//   each lane then holds four consecutive output columns of one activation
//   row, which the epilogue packs to 8-byte LDS writes; the finished tile
//   leaves through LDS as coalesced 16-byte global stores.
// * operands are read through range-checked buffer resource descriptors:
//   rows beyond the group and the K tail go to an out-of-range offset and
//   read as zeros, so no lane branches and no select waits on loaded data.
#include "moe_internal.h"

namespace moe {

hipError_t launch_schedule(const moe_desc &d, const int32_t *offsets, int32_t *mtile_start,
                           int bm, hipStream_t s);

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));  // one 16-byte chunk
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

enum { EPI_SWIGLU = 0, EPI_SILU_BIAS = 1, EPI_BIAS = 2, EPI_GELU_BIAS = 3 };

struct GemmParams {
    const __bf16 *A;              // x (gathered rows) or H (dispatch rows)
    int32_t a_bytes;              // bytes of x (< 2^31, checked on the host); unused for H
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

// Raw buffer resource over [base, base + bytes): the 4th descriptor word is
// the gfx9-family default (32-bit dwords, no swizzle); loads at offsets >=
// bytes return zero.
constexpr int kRsrcWord3 = 0x00020000;
constexpr int kOOB = (int)0x80000000u;  // an offset beyond every resource (< 2^31 bytes)

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void *base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(base), (short)0, bytes, kRsrcWord3);
}

// Values every lane of a wave shares but that the compiler cannot prove
// uniform (they come from LDS or from memory indexed by LDS values).  Taking
// them through readfirstlane keeps the derived pointers and buffer resources in
// scalar registers; otherwise each buffer load with such a resource is wrapped
// in a per-lane loop.
__device__ __forceinline__ int wave_uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }

__device__ __forceinline__ float silu_fast(float z) {
    return z * __builtin_amdgcn_rcpf(1.0f + __expf(-z));
}

// exact GELU, z * Phi(z), with the device library's erff
__device__ __forceinline__ float gelu_exact(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

template <int BM, int BN, int WM, int WN>
struct TileCfg {
    static constexpr int BK = 64;  // 8 chunks of 16 bytes per LDS row
    static constexpr int TILE_M = BM;
    static constexpr int NTH = WM * WN * 64;
    static constexpr int WTM = BM / WM, WTN = BN / WN;  // wave tile (x rows, weight rows)
    static constexpr int FM = WTM / 32, FN = WTN / 32;   // 32x32 fragments per wave
    static constexpr int RPP = NTH / 8;                  // tile rows per load pass
    static constexpr int A_LD = BM / RPP, B_LD = BN / RPP;
    static_assert(BM % RPP == 0 && BN % RPP == 0, "tile / thread mismatch");
    static_assert(FM >= 1 && FN >= 1, "wave tile");
};

template <int BM, int BN, int BNO>
struct Smem {
    static constexpr int kOperand = 2 * (BM + BN) * 8 * 16;         // double-buffered A and B
    static constexpr int kPitch = BNO * 2 + 16;                     // epilogue row pitch, bytes
    static constexpr int kEpilogue = BM * kPitch;
    static constexpr int kBytes = kOperand > kEpilogue ? kOperand : kEpilogue;
};

template <int BM, int BN, int WM, int WN, int EPI, bool GATHER>
__global__ __launch_bounds__(WM *WN * 64) void grouped_gemm_bf16_kernel(GemmParams p) {
    typedef TileCfg<BM, BN, WM, WN> C;
    constexpr int BK = C::BK, NTH = C::NTH, WTM = C::WTM, WTN = C::WTN;
    constexpr int FM = C::FM, FN = C::FN, RPP = C::RPP, A_LD = C::A_LD, B_LD = C::B_LD;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int BNO = GATED ? BN / 2 : BN;  // output columns per tile
    static_assert(!GATED || FN % 2 == 0, "SwiGLU needs act/lin fragment pairs");
    typedef Smem<BM, BN, BNO> S;

    __shared__ __attribute__((aligned(16))) unsigned char smem[S::kBytes];
    __shared__ int s_start[kMaxGroups + 1];
    u32x4 *sA = reinterpret_cast<u32x4 *>(smem);           // [2][BM * 8]
    u32x4 *sB = sA + 2 * BM * 8;                           // [2][BN * 8]

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm = wave / WN, wn = wave % WN;

    for (int g = tid; g <= p.G; g += NTH) s_start[g] = p.mtile_start[g];
    __syncthreads();

    // ---- tile of this workgroup (XCD-aware order) --------------------------
    const int ntn = (p.N + BNO - 1) / BNO;
    const int total = wave_uniform(s_start[p.G]) * ntn;
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
    const int g = wave_uniform(lo);
    const bool shared = g >= p.E;
    const int64_t grow0 = shared ? 0 : wave_uniform(p.offsets[g]);
    const int64_t M = shared ? p.T : (int64_t)wave_uniform(p.offsets[g + 1]) - grow0;
    const int64_t m0 = (int64_t)(mt - wave_uniform(s_start[g])) * BM;
    const int64_t crow0 = shared ? p.shared_row0 : grow0;
    const int n0 = nt * BNO;
    const int N = p.N, K = p.K;
    const int64_t wstride = (int64_t)N * K;
    const __bf16 *W0 = shared ? p.Ws0 : p.W0 + g * wstride;
    const __bf16 *W1 = GATED ? (shared ? p.Ws1 : p.W1 + g * wstride) : nullptr;
    const __bf16 *bias = EPI == EPI_SWIGLU ? nullptr
                         : shared         ? p.bs
                         : (p.bias ? p.bias + (int64_t)g * N : nullptr);

    // ---- operand resources and per-thread byte offsets ---------------------
    const int cq = tid & 7;  // 16-byte chunk within a 64-wide K slice
    // A: gathered rows of x through one descriptor over x, or this tile's
    // own contiguous rows of H through a descriptor based at its first row
    // (so H as a whole may exceed the 2 GiB a 32-bit offset reaches)
    const __bf16 *abase = GATHER ? p.A : p.A + (crow0 + m0) * K;
    const int abytes = GATHER ? p.a_bytes : (int)(min((int64_t)BM, M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(abase, abytes);
    const __amdgpu_buffer_rsrc_t rW0 = make_rsrc(W0, (int)(wstride * 2));
    const __amdgpu_buffer_rsrc_t rW1 = make_rsrc(GATED ? W1 : W0, (int)(wstride * 2));
    int a_off[A_LD];  // byte offset of this thread's chunk in its A row, or kOOB
#pragma unroll
    for (int i = 0; i < A_LD; ++i) {
        const int r = (tid >> 3) + i * RPP;
        const int64_t lr = m0 + r;
        if (lr < M) {
            const int64_t src = GATHER ? (shared ? lr : (int64_t)p.sorted_token[grow0 + lr]) : r;
            a_off[i] = (int)(src * K * 2) + cq * 16;
        } else {
            a_off[i] = kOOB;
        }
    }
    int b_off[B_LD];  // byte offset in W_act (or, for the second half of a SwiGLU tile, W_lin)
#pragma unroll
    for (int i = 0; i < B_LD; ++i) {
        const int r = (tid >> 3) + i * RPP;
        const int n = n0 + ((GATED && r >= BN / 2) ? r - BN / 2 : r);
        b_off[i] = n < N ? n * K * 2 + cq * 16 : kOOB;
    }

    const int KT = (K + BK - 1) / BK;
    u32x4 ra[A_LD], rb[B_LD];

#define MOE_GLOAD(KTILE)                                                              \
    {                                                                                 \
        const int kc = (KTILE) * BK + cq * 8;                                         \
        const int kb = kc < K ? (KTILE) * BK * 2 : kOOB;                              \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i)                              \
            ra[i] = __builtin_amdgcn_raw_buffer_load_b128(                            \
                rA, a_off[i] == kOOB || kb == kOOB ? kOOB : a_off[i] + kb, 0, 0);     \
        _Pragma("unroll") for (int i = 0; i < B_LD; ++i) {                            \
            const int off = b_off[i] == kOOB || kb == kOOB ? kOOB : b_off[i] + kb;    \
            rb[i] = (GATED && (i * RPP >= BN / 2))                                    \
                        ? __builtin_amdgcn_raw_buffer_load_b128(rW1, off, 0, 0)       \
                        : __builtin_amdgcn_raw_buffer_load_b128(rW0, off, 0, 0);      \
        }                                                                             \
    }
#define MOE_SSTORE(BUF)                                                               \
    {                                                                                 \
        u32x4 *dA = sA + (BUF) * BM * 8;                                              \
        u32x4 *dB = sB + (BUF) * BN * 8;                                              \
        _Pragma("unroll") for (int i = 0; i < A_LD; ++i) {                            \
            const int r = (tid >> 3) + i * RPP;                                       \
            dA[r * 8 + (cq ^ swz(r))] = ra[i];                                        \
        }                                                                             \
        _Pragma("unroll") for (int i = 0; i < B_LD; ++i) {                            \
            const int r = (tid >> 3) + i * RPP;                                       \
            dB[r * 8 + (cq ^ swz(r))] = rb[i];                                        \
        }                                                                             \
    }

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // LDS rows of this wave's fragments: x rows (MFMA columns) and weight rows
    // (MFMA rows); for SwiGLU the first FN/2 weight fragments are W_act rows,
    // the rest the matching W_lin rows.
    int xrow[FM], wrow[FN];
#pragma unroll
    for (int j = 0; j < FM; ++j) xrow[j] = wm * WTM + j * 32 + (lane & 31);
#pragma unroll
    for (int i = 0; i < FN; ++i) {
        if (GATED)
            wrow[i] = (i < FN / 2 ? wn * (WTN / 2) + i * 32
                                  : BN / 2 + wn * (WTN / 2) + (i - FN / 2) * 32) + (lane & 31);
        else
            wrow[i] = wn * WTN + i * 32 + (lane & 31);
    }
    const int khalf = lane >> 5;

    MOE_GLOAD(0);
    MOE_SSTORE(0);
    __syncthreads();
    for (int kt = 0; kt < KT; ++kt) {
        const int buf = kt & 1;
        if (kt + 1 < KT) MOE_GLOAD(kt + 1);
        const u32x4 *cA = sA + buf * BM * 8;
        const u32x4 *cB = sB + buf * BN * 8;
        bf16x8 fw[2][FN], fx[2][FM];
#pragma unroll
        for (int kk = 0; kk < BK / 16; ++kk) {
            const int cur = kk & 1;
            if (kk == 0) {
                const int ch = khalf;
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    fw[0][i] = __builtin_bit_cast(bf16x8, cB[wrow[i] * 8 + (ch ^ swz(wrow[i]))]);
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    fx[0][j] = __builtin_bit_cast(bf16x8, cA[xrow[j] * 8 + (ch ^ swz(xrow[j]))]);
            }
            if (kk + 1 < BK / 16) {  // next K step's fragments while this step's MFMAs run
                const int ch = (kk + 1) * 2 + khalf;
#pragma unroll
                for (int i = 0; i < FN; ++i)
                    fw[cur ^ 1][i] = __builtin_bit_cast(bf16x8, cB[wrow[i] * 8 + (ch ^ swz(wrow[i]))]);
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    fx[cur ^ 1][j] = __builtin_bit_cast(bf16x8, cA[xrow[j] * 8 + (ch ^ swz(xrow[j]))]);
            }
#pragma unroll
            for (int i = 0; i < FN; ++i)
#pragma unroll
                for (int j = 0; j < FM; ++j)
                    acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fw[cur][i], fx[cur][j],
                                                                        acc[i][j], 0, 0, 0);
        }
        if (kt + 1 < KT) MOE_SSTORE(buf ^ 1);
        __syncthreads();
    }
#undef MOE_GLOAD
#undef MOE_SSTORE

    // ---- epilogue: activation, bf16, staged through LDS ---------------------
    // acc[i][j][v]: weight row 8*(v/4) + 4*(lane/32) + (v%4) of fragment i,
    // activation row (lane & 31) of fragment j.  The operand buffers are free
    // after the final barrier of the K loop.
    unsigned char *ctile = smem;
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + j * 32 + (lane & 31);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            if (GATED) {
#pragma unroll
                for (int i = 0; i < FN / 2; ++i) {
                    const int nl = wn * (WTN / 2) + i * 32 + gq * 8 + khalf * 4;
                    bf16x4 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q)
                        h[q] = (__bf16)(silu_fast(acc[i][j][gq * 4 + q]) * acc[i + FN / 2][j][gq * 4 + q]);
                    *reinterpret_cast<bf16x4 *>(ctile + ml * S::kPitch + nl * 2) = h;
                }
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int nl = wn * WTN + i * 32 + gq * 8 + khalf * 4;
                    bf16x4 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int n = n0 + nl + q;
                        float v = acc[i][j][gq * 4 + q];
                        if (bias) v += (float)bias[n < N ? n : 0];
                        if (EPI == EPI_SILU_BIAS) v = silu_fast(v);
                        if (EPI == EPI_GELU_BIAS) v = gelu_exact(v);
                        h[q] = (__bf16)v;
                    }
                    *reinterpret_cast<bf16x4 *>(ctile + ml * S::kPitch + nl * 2) = h;
                }
            }
        }
    }
    __syncthreads();
    constexpr int CPR = BNO / 8;  // 16-byte chunks per tile row
    for (int c = tid; c < BM * CPR; c += NTH) {
        const int ml = c / CPR;
        const int ch = c - ml * CPR;
        const int64_t lr = m0 + ml;
        const int n = n0 + ch * 8;
        if (lr < M && n < N) {
            const u32x4 v = *reinterpret_cast<const u32x4 *>(ctile + ml * S::kPitch + ch * 16);
            *reinterpret_cast<u32x4 *>(p.C + (crow0 + lr) * N + n) = v;
        }
    }
}

#define MOE_LDS(p) ((__attribute__((address_space(3))) void *)(p))

// ---------------------------------------------------------------------------
// Five half-stage form: K slices of 64 (one 128-byte line per row and load,
// as in the two-stage form), but each slice is split into its activation
// half (A, 256 rows x 128 bytes) and its weight half (B, the same), and the
// halves rotate through five 32 KiB slots -- all 160 KiB of LDS.  At slice s
// the A half of s+1 and the B half of s+2 are requested, so weights (the
// HBM-bound operand) are fetched two slices ahead and activations one, 96 KiB
// in flight.  Half h (B of slice s: h = 2s, A of slice s: h = 2s+1) lives in
// slot h mod 5; the loop is unrolled five slices deep with an exit after each
// slice.  The group table sits in slot 4 until the first load into it.
// ---------------------------------------------------------------------------
namespace r5 {
// M tiles per band of a group's tile order: the N tiles of a band run one
// after another, each over the band's M tiles.  Measured against M-tile-major
// order: Mixtral expert stage 11.34 -> 10.05 ms, DeepSeek prefill 5.92 ->
// 5.76 ms, headline unchanged (bands of 4: 10.19 / 5.74 ms).
constexpr int kBandM = 8;
constexpr int BM = 256, BN = 256, WM = 2, WN = 4, NTH = 512, BK = 64;
constexpr int WTM = BM / WM, WTN = BN / WN, FM = WTM / 32, FN = WTN / 32;
constexpr int CH = BK * 2 / 16;   // 16-byte chunks per LDS row (8)
constexpr int SLOT = BM * CH;     // chunks per half-stage slot (2048 = 32 KiB)
static_assert(BM == BN, "A and B halves share the slot size");

__device__ __forceinline__ bf16x8 lds_frag(const char *base, int off) {
    return __builtin_bit_cast(bf16x8, *reinterpret_cast<const u32x4 *>(base + off));
}

// Fragment q of a k step: q < FN is weight fragment q, else activation
// fragment q - FN.
template <int BSTEP>
__device__ __forceinline__ void frag_read(int q, bf16x8 (&fw)[FN], bf16x8 (&fx)[FM],
                                          const char *sa, int ao, const char *sb, int bo) {
    if (q < FN) fw[q] = lds_frag(sb, bo + q * BSTEP);
    else fx[q - FN] = lds_frag(sa, ao + (q - FN) * 32 * CH * 16);
}

// The products of one k step (fragments P) with the fragment reads of the
// next step (into Q) issued between them, one read after each product.
template <int BSTEP>
__device__ __forceinline__ void kstep(f32x16 (&acc)[FN][FM], const bf16x8 (&fwP)[FN],
                                      const bf16x8 (&fxP)[FM], bf16x8 (&fwQ)[FN],
                                      bf16x8 (&fxQ)[FM], const char *sa, int ao,
                                      const char *sb, int bo) {
    constexpr int NM = FN * FM, ND = FN + FM;
#pragma unroll
    for (int t = 0; t < NM; ++t) {
        const int i = t / FM, j = t % FM;
        acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fwP[i], fxP[j], acc[i][j], 0, 0, 0);
        if (t < ND) frag_read<BSTEP>(t, fwQ, fxQ, sa, ao, sb, bo);
    }
#pragma unroll
    for (int t = NM; t < ND; ++t) frag_read<BSTEP>(t, fwQ, fxQ, sa, ao, sb, bo);
}

// Issue order of one k step's fragment reads (DS) and products (MFMA) for
// the machine scheduler: eight products with the six reads of the next step
// placed one after each product.
__device__ __forceinline__ void pin_step_order() {
#pragma unroll
    for (int t = 0; t < FN + FM; ++t) {
        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
        __builtin_amdgcn_sched_group_barrier(0x100, 1, 0);
    }
    __builtin_amdgcn_sched_group_barrier(0x008, FN * FM - (FN + FM), 0);
}
}  // namespace r5

template <int EPI, bool GATHER>
__global__ __launch_bounds__(512) void grouped_gemm_r5_kernel(GemmParams p) {
    using namespace r5;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int BNO = GATED ? BN / 2 : BN;
    static_assert(!GATED || FN == 2, "one W_act and one W_lin fragment per wave");
    __shared__ __attribute__((aligned(16))) u32x4 st0[SLOT];
    __shared__ __attribute__((aligned(16))) u32x4 st1[SLOT];
    __shared__ __attribute__((aligned(16))) u32x4 st2[SLOT];
    __shared__ __attribute__((aligned(16))) u32x4 st3[SLOT];
    __shared__ __attribute__((aligned(16))) u32x4 st4[SLOT];
    int *s_start = reinterpret_cast<int *>(st4);  // until slot 4's first load
    static_assert((kMaxGroups + 1) * 4 <= SLOT * 16, "group table fits in a slot");

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);
    const int wm = wave / WN, wn = wave % WN;
    const int khalf = lane >> 5;

    for (int g = tid; g <= p.G; g += NTH) s_start[g] = p.mtile_start[g];
    __syncthreads();

    // ---- tile of this workgroup (XCD-aware order) --------------------------
    const int ntn = (p.N + BNO - 1) / BNO;
    const int total = wave_uniform(s_start[p.G]) * ntn;
    const int per_xcd = (total + 7) >> 3;
    const int slot8 = blockIdx.x >> 3;
    if (slot8 >= per_xcd) return;
    const int logical = (blockIdx.x & 7) * per_xcd + slot8;
    if (logical >= total) return;
    // group g owns logical tiles [s_start[g] * ntn, s_start[g+1] * ntn)
    const int mt = logical / ntn;
    int lo = 0, hi = p.G - 1;
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (s_start[mid] <= mt) lo = mid; else hi = mid - 1;
    }
    const int g = wave_uniform(lo);
    const int mt0 = wave_uniform(s_start[g]);
    // inside the group, bands of GROUP_M M tiles: the N tiles of a band run
    // one after another, each over the band's M tiles, so tiles that share a
    // weight panel start within a few tiles of each other (and those sharing
    // an activation panel within GROUP_M) while the panel is still in L2
    const int nmt = wave_uniform(s_start[g + 1]) - mt0;
    const int li = logical - mt0 * ntn;
    const int band = li / (r5::kBandM * ntn);
    const int rem = li - band * r5::kBandM * ntn;
    const int rows = min(r5::kBandM, nmt - band * r5::kBandM);
    const int nt = rem / rows;
    const int mtl = band * r5::kBandM + rem - nt * rows;
    const bool shared = g >= p.E;
    const int64_t grow0 = shared ? 0 : wave_uniform(p.offsets[g]);
    const int64_t M = shared ? p.T : (int64_t)wave_uniform(p.offsets[g + 1]) - grow0;
    const int64_t m0 = (int64_t)mtl * BM;
    const int64_t crow0 = shared ? p.shared_row0 : grow0;
    const int n0 = nt * BNO;
    const int N = p.N, K = p.K;
    const int64_t wstride = (int64_t)N * K;
    const __bf16 *W0 = shared ? p.Ws0 : p.W0 + g * wstride;
    const __bf16 *W1 = GATED ? (shared ? p.Ws1 : p.W1 + g * wstride) : W0;
    const __bf16 *bias = EPI == EPI_SWIGLU ? nullptr
                         : shared         ? p.bs
                         : (p.bias ? p.bias + (int64_t)g * N : nullptr);
    // A: gathered rows of x through one descriptor over x, or this tile's
    // own contiguous rows of H through a descriptor based at its first row
    // (so H as a whole may exceed the 2 GiB a 32-bit offset reaches)
    const __bf16 *abase = GATHER ? p.A : p.A + (crow0 + m0) * K;
    const int abytes = GATHER ? p.a_bytes : (int)(min((int64_t)BM, M - m0) * K * 2);
    const __amdgpu_buffer_rsrc_t rA = make_rsrc(abase, abytes);
    const __amdgpu_buffer_rsrc_t rB = make_rsrc(GATED && wave >= 4 ? W1 : W0, (int)(wstride * 2));

    // ---- DMA: load j of a lane covers row (4*wave + j)*8 + lane/8 of a half
    // and LDS slot lane%8 of it, which holds logical chunk (lane%8) ^ swz(row)
    int a_off[4], b_off[4], kc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = (4 * wave + j) * 8 + (lane >> 3);
        const int c = (lane & 7) ^ swz(r);
        kc[j] = c * 8;
        const int64_t lr = m0 + r;
        if (lr < M) {
            const int64_t src = GATHER ? (shared ? lr : (int64_t)p.sorted_token[grow0 + lr]) : r;
            a_off[j] = (int)(src * K * 2) + c * 16;
        } else {
            a_off[j] = kOOB;
        }
        const int rn = GATED && r >= BN / 2 ? r - BN / 2 : r;
        b_off[j] = n0 + rn < N ? (n0 + rn) * K * 2 + c * 16 : kOOB;
    }
    const int KT = (K + BK - 1) / BK;

#define MOE_R5_ISSUE(STG, RS, OFF, Q)                                                        \
    {                                                                                        \
        const int q_ = (Q);                                                                  \
        _Pragma("unroll") for (int j = 0; j < 4; ++j) {                                      \
            const bool ok = q_ * BK + kc[j] < K && OFF[j] != kOOB;                           \
            __builtin_amdgcn_raw_ptr_buffer_load_lds(                                        \
                RS, MOE_LDS((STG) + (4 * wave + j) * 64), 16, ok ? OFF[j] + q_ * BK * 2 : kOOB, \
                0, 0, 0);                                                                    \
        }                                                                                    \
    }

    f32x16 acc[FN][FM];
#pragma unroll
    for (int i = 0; i < FN; ++i)
#pragma unroll
        for (int j = 0; j < FM; ++j)
#pragma unroll
            for (int v = 0; v < 16; ++v) acc[i][j][v] = 0.f;

    // Fragment addressing.  Every fragment row is a multiple of 32 plus
    // lane % 32, so all rows of a lane share one swizzle, and one byte offset
    // per 16-wide k step serves every fragment: activation fragment j sits
    // 4 KiB further per j, weight fragment i BSTEP further per i.
    constexpr int BSTEP = GATED ? (BN / 2) * CH * 16 : 32 * CH * 16;
    int aofs[4], bofs[4];
    {
        const int l32 = lane & 31;
        const int sw = swz(l32);
#pragma unroll
        for (int ks = 0; ks < 4; ++ks) {
            const int lo = l32 * CH * 16 + (((2 * ks + khalf) ^ sw) << 4);
            aofs[ks] = wm * WTM * CH * 16 + lo;
            bofs[ks] = (GATED ? wn * (WTN / 2) : wn * WTN) * CH * 16 + lo;
        }
    }
    // a wave whose 128 rows all lie past the group's end (zeros) skips its
    // fragment reads and products: one uniform branch per slice.  Partly
    // live waves multiply the zero rows too -- per-product branches, or one
    // K-loop copy per live count, cost more than they save (the copies
    // exhaust the registers).
    const bool live = m0 + wm * WTM < M;

    // The products of a slice's last k step run after the barrier that ends
    // the slice, with the first reads of the next slice placed between them:
    // no wave waits for fragments at the start of a slice.  Before the first
    // slice the held step is zeros (its products add nothing).
    bf16x8 fwX[FN], fxX[FM], fwY[FN], fxY[FM];
#pragma unroll
    for (int i = 0; i < FN; ++i) fwY[i] = bf16x8{};
#pragma unroll
    for (int j = 0; j < FM; ++j) fxY[j] = bf16x8{};
    // slice s: B half in SB, A half in SA; requests A of s+1 into IA and B of
    // s+2 into IB (both slots were read to the end in slice s-1); multiplies
    // the held last step of s-1 while reading step 0 of s, then steps 0-2 of s
    // while reading steps 1-3.  At the end every half of slice s+1 has landed
    // (vmcnt(4) leaves only B of s+2) and the reads of step 3 are in
    // registers.  The offsets pass through an empty asm so that their sums
    // with the slot addresses are formed in the slice, not held in registers
    // across the loop.
#define MOE_R5_SLICE(SB, SA, IA, IB, S)                                                      \
    {                                                                                        \
        int ao0 = aofs[0], ao1 = aofs[1], ao2 = aofs[2], ao3 = aofs[3];                      \
        int bo0 = bofs[0], bo1 = bofs[1], bo2 = bofs[2], bo3 = bofs[3];                      \
        asm volatile("" : "+v"(ao0), "+v"(ao1), "+v"(ao2), "+v"(ao3), "+v"(bo0),             \
                     "+v"(bo1), "+v"(bo2), "+v"(bo3));                                       \
        const char *sa_ = reinterpret_cast<const char *>(SA);                                \
        const char *sb_ = reinterpret_cast<const char *>(SB);                                \
        MOE_R5_ISSUE(IA, rA, a_off, (S) + 1);                                                \
        if (live) {                                                                          \
            r5::kstep<BSTEP>(acc, fwY, fxY, fwX, fxX, sa_, ao0, sb_, bo0);                   \
            r5::pin_step_order();                                                            \
        }                                                                                    \
        MOE_R5_ISSUE(IB, rB, b_off, (S) + 2);                                                \
        if (live) {                                                                          \
            r5::kstep<BSTEP>(acc, fwX, fxX, fwY, fxY, sa_, ao1, sb_, bo1);                   \
            r5::kstep<BSTEP>(acc, fwY, fxY, fwX, fxX, sa_, ao2, sb_, bo2);                   \
            r5::kstep<BSTEP>(acc, fwX, fxX, fwY, fxY, sa_, ao3, sb_, bo3);                   \
            r5::pin_step_order();                                                            \
            r5::pin_step_order();                                                            \
            r5::pin_step_order();                                                            \
        }                                                                                    \
        __builtin_amdgcn_sched_barrier(0);                                                   \
        __builtin_amdgcn_s_waitcnt(0x0074); /* vmcnt(4) lgkmcnt(0) */                        \
        __builtin_amdgcn_s_barrier();                                                        \
        asm volatile("" ::: "memory");                                                       \
        __builtin_amdgcn_sched_barrier(0);                                                   \
    }
    // prologue: B0 -> slot 0, A0 -> slot 1, B1 -> slot 2; wait for B0 and A0
    MOE_R5_ISSUE(st0, rB, b_off, 0);
    MOE_R5_ISSUE(st1, rA, a_off, 0);
    MOE_R5_ISSUE(st2, rB, b_off, 1);
    asm volatile("" ::: "memory");  // the group table is read before this point
    __builtin_amdgcn_s_waitcnt(0x0074);
    __builtin_amdgcn_s_barrier();  // also: every wave is done with the group table
    asm volatile("" ::: "memory");
    for (int s = 0;;) {
        MOE_R5_SLICE(st0, st1, st3, st4, s)
        if (++s >= KT) break;
        MOE_R5_SLICE(st2, st3, st0, st1, s)
        if (++s >= KT) break;
        MOE_R5_SLICE(st4, st0, st2, st3, s)
        if (++s >= KT) break;
        MOE_R5_SLICE(st1, st2, st4, st0, s)
        if (++s >= KT) break;
        MOE_R5_SLICE(st3, st4, st1, st2, s)
        if (++s >= KT) break;
    }
    if (live) {  // the held last step of the last slice
#pragma unroll
        for (int i = 0; i < FN; ++i)
#pragma unroll
            for (int j = 0; j < FM; ++j)
                acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(fwY[i], fxY[j], acc[i][j], 0, 0, 0);
    }
    __builtin_amdgcn_s_waitcnt(0x0070);  // drain the look-ahead loads past K
    __syncthreads();
#undef MOE_R5_SLICE
#undef MOE_R5_ISSUE

    // ---- epilogue, staged through slots 0-3 as whole output rows ------------
    constexpr int CPR = BNO / 8;     // 16-byte chunks per output row
    constexpr int RPS = SLOT / CPR;  // tile rows per slot
    static_assert(RPS * 4 >= BM, "the output tile fits in four slots");
#pragma unroll
    for (int j = 0; j < FM; ++j) {
        const int ml = wm * WTM + j * 32 + (lane & 31);
        const int sidx = ml / RPS;
        u32x4 *stg = sidx == 0 ? st0 : sidx == 1 ? st1 : sidx == 2 ? st2 : st3;
        char *rowp = reinterpret_cast<char *>(stg + (ml % RPS) * CPR);
#pragma unroll
        for (int gq = 0; gq < 4; ++gq) {
            if (GATED) {
                const int nl = wn * (WTN / 2) + gq * 8 + khalf * 4;
                bf16x4 h;
#pragma unroll
                for (int q = 0; q < 4; ++q)
                    h[q] = (__bf16)(silu_fast(acc[0][j][gq * 4 + q]) * acc[1][j][gq * 4 + q]);
                *reinterpret_cast<bf16x4 *>(rowp + (((nl >> 3) ^ (ml & (CPR - 1))) << 4) + khalf * 8) = h;
            } else {
#pragma unroll
                for (int i = 0; i < FN; ++i) {
                    const int nl = wn * WTN + i * 32 + gq * 8 + khalf * 4;
                    const int n = n0 + nl;
                    bf16x4 h;
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        float v = acc[i][j][gq * 4 + q];
                        if (bias && n < N) v += (float)bias[n + q];
                        if (EPI == EPI_SILU_BIAS) v = silu_fast(v);
                        if (EPI == EPI_GELU_BIAS) v = gelu_exact(v);
                        h[q] = (__bf16)v;
                    }
                    *reinterpret_cast<bf16x4 *>(rowp + (((nl >> 3) ^ (ml & (CPR - 1))) << 4) + khalf * 8) = h;
                }
            }
        }
    }
    __syncthreads();
    {
        const int c = tid % CPR;
        const int n = n0 + c * 8;
        if (n < N) {
#pragma unroll 4
            for (int r = tid / CPR; r < BM; r += NTH / CPR) {
                const int64_t lr = m0 + r;
                if (lr >= M) break;
                const u32x4 *stg = r < RPS ? st0 : r < 2 * RPS ? st1 : r < 3 * RPS ? st2 : st3;
                const u32x4 v = stg[(r % RPS) * CPR + (c ^ (r & (CPR - 1)))];
                *reinterpret_cast<u32x4 *>(p.C + (crow0 + lr) * N + n) = v;
            }
        }
    }
}

template <int EPI, bool GATHER>
hipError_t launch_r5(const GemmParams &p, int64_t max_mtiles, hipStream_t s) {
    constexpr int BNO = EPI == EPI_SWIGLU ? r5::BN / 2 : r5::BN;
    const int64_t ntn = ceil_div(p.N, BNO);
    const int64_t blocks = ceil_div(max_mtiles * ntn, 8) * 8;
    if (blocks == 0) return hipSuccess;
    grouped_gemm_r5_kernel<EPI, GATHER><<<(unsigned)blocks, r5::NTH, 0, s>>>(p);
    return hipGetLastError();
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

// "Narrow" register-staged tiles for a handful of rows per expert (decode),
// where the stage streams weights from HBM and more, smaller workgroups keep
// more bytes in flight; the five-slot kernel above for everything else.
// 32-row tiles of 256 weight rows, one wave row of four waves: the decode
// expert stage streams its touched weights at the part's practical rate with
// this shape (deeper register prefetch changed nothing).
constexpr int kNarrowBM = 32, kNarrowBN = 256, kNarrowWM = 1, kNarrowWN = 4;
// Mean kept rows per routed expert below which the narrow tiles are used:
// at 48 rows a 256-row tile is under a fifth full and the wide kernel's
// decode expert stage took 2325 us against 2152-2163 us for the narrow one.
constexpr int kNarrowMaxRows = 48;

template <int BM, int BN, int WM, int WN>
hipError_t run_ffn(const moe_desc &d, const GemmParams &up, const GemmParams &dn,
                   int32_t *mtile_start, int64_t rows_routed_max, hipStream_t s,
                   bool schedule_ready) {
    hipError_t e = schedule_ready ? hipSuccess : launch_schedule(d, up.offsets, mtile_start, BM, s);
    if (e != hipSuccess) return e;
    // upper bound of the M tiles: sum_g ceil(rows_g / BM) <= ceil(R / BM) + E
    const int64_t max_mtiles = ceil_div(rows_routed_max, BM) +
                               std::min<int64_t>(d.E, rows_routed_max) +
                               (d.n_shared ? ceil_div(d.T, BM) : 0);
    if (d.expert_kind == MOE_EXPERT_SWIGLU) e = launch_one<BM, BN, WM, WN, EPI_SWIGLU, true>(up, max_mtiles, s);
    else if (d.expert_kind == MOE_EXPERT_GELU_MLP) e = launch_one<BM, BN, WM, WN, EPI_GELU_BIAS, true>(up, max_mtiles, s);
    else e = launch_one<BM, BN, WM, WN, EPI_SILU_BIAS, true>(up, max_mtiles, s);
    if (e != hipSuccess) return e;
    return launch_one<BM, BN, WM, WN, EPI_BIAS, false>(dn, max_mtiles, s);
}

hipError_t run_ffn_wide(const moe_desc &d, const GemmParams &up, const GemmParams &dn,
                        int32_t *mtile_start, int64_t rows_routed_max, hipStream_t s,
                        bool schedule_ready) {
    constexpr int BM = r5::BM;
    hipError_t e = schedule_ready ? hipSuccess : launch_schedule(d, up.offsets, mtile_start, BM, s);
    if (e != hipSuccess) return e;
    const int64_t max_mtiles = ceil_div(rows_routed_max, BM) +
                               std::min<int64_t>(d.E, rows_routed_max) +
                               (d.n_shared ? ceil_div(d.T, BM) : 0);
    if (d.expert_kind == MOE_EXPERT_SWIGLU) e = launch_r5<EPI_SWIGLU, true>(up, max_mtiles, s);
    else if (d.expert_kind == MOE_EXPERT_GELU_MLP) e = launch_r5<EPI_GELU_BIAS, true>(up, max_mtiles, s);
    else e = launch_r5<EPI_SILU_BIAS, true>(up, max_mtiles, s);
    if (e != hipSuccess) return e;
    return launch_r5<EPI_BIAS, false>(dn, max_mtiles, s);
}

}  // namespace

static bool use_narrow(const moe_desc &d, const Workspace &w) {
    return w.rows_routed_max < (int64_t)kNarrowMaxRows * d.E;
}

int grouped_ffn_bm(const moe_desc &d, const Workspace &w) {
    if (d.dtype != MOE_BF16) return kGemmBMf32;
    if (use_narrow(d, w)) return TileCfg<kNarrowBM, kNarrowBN, kNarrowWM, kNarrowWN>::TILE_M;
    return r5::BM;
}

// Up projection (+ activation) then down projection for every group.
hipError_t launch_grouped_ffn_bf16(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                                   const ExpertArgs &a, hipStream_t s, bool schedule_ready) {
    __bf16 *H = reinterpret_cast<__bf16 *>(a.ws + w.H);
    int32_t *mtile_start = reinterpret_cast<int32_t *>(a.ws + w.mtile_start);
    GemmParams up{};
    up.A = (const __bf16 *)a.x;
    up.a_bytes = (int32_t)(d.T * d.d_model * 2);
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
    GemmParams dn = up;
    dn.A = H;
    dn.a_bytes = 0;  // each tile's descriptor covers its own rows of H
    dn.W0 = (const __bf16 *)wt.w_down;
    dn.W1 = nullptr;
    dn.bias = (const __bf16 *)wt.b_down;
    dn.Ws0 = (const __bf16 *)wt.ws_down;
    dn.Ws1 = nullptr;
    dn.bs = (const __bf16 *)wt.bs_down;
    dn.C = (__bf16 *)a.Y;
    dn.N = d.d_model;
    dn.K = d.d_ff;
    if (use_narrow(d, w))
        return run_ffn<kNarrowBM, kNarrowBN, kNarrowWM, kNarrowWN>(d, up, dn, mtile_start, w.rows_routed_max, s, schedule_ready);
    return run_ffn_wide(d, up, dn, mtile_start, w.rows_routed_max, s, schedule_ready);
}

}  // namespace moe
