// K3 (f32): grouped expert GEMM in float32 on the vector ALUs.
//
// Same grouped schedule and epilogues as the bf16 matrix-core kernel (the
// SiLU MLP with biases of Expert Networks > Code Implementation, In[7]; the
// SwiGLU of the LLMs-from-scratch MoE guide, "Expert forward pass"), for
// float32 layers, whose 1e-5 tolerance rules out reduced-precision matrix
// math.  A classic LDS-tiled SGEMM: 64 x 64 output tile, K slices of 16,
// 256 threads with a 4 x 4 register micro-tile each (plus the matching 4 x 4
// of the linear branch for SwiGLU), f32 fused multiply-add accumulation.
#include "moe_internal.h"

namespace moe {

hipError_t launch_schedule(const moe_desc &d, const int32_t *offsets, int32_t *mtile_start,
                           int bm, hipStream_t s);

namespace {

enum { EPI_SWIGLU = 0, EPI_SILU_BIAS = 1, EPI_BIAS = 2, EPI_GELU_BIAS = 3 };

struct GemmParamsF32 {
    const float *A;
    const int32_t *sorted_token;
    const int32_t *offsets;
    const int32_t *mtile_start;
    const float *W0, *W1, *bias;
    const float *Ws0, *Ws1, *bs;
    float *C;
    int64_t T;
    int64_t shared_row0;
    int E, G, N, K;
};

__device__ __forceinline__ float silu_exact(float z) { return z / (1.0f + expf(-z)); }
// exact GELU, z * Phi(z), with the device library's erff
__device__ __forceinline__ float gelu_exact(float z) {
    return 0.5f * z * (1.0f + erff(z * 0.70710678118654752f));
}

template <int EPI, bool GATHER>
__global__ __launch_bounds__(256) void grouped_gemm_f32_kernel(GemmParamsF32 p) {
    constexpr int BM = kGemmBMf32, BNO = 64, BK = 16;
    constexpr bool GATED = EPI == EPI_SWIGLU;
    constexpr int BNB = GATED ? 2 * BNO : BNO;  // weight rows per tile
    __shared__ float As[BK][BM + 4];
    __shared__ float Bs[BK][BNB + 4];
    __shared__ int s_start[kMaxGroups + 1];

    const int tid = threadIdx.x;
    for (int g = tid; g <= p.G; g += 256) s_start[g] = p.mtile_start[g];
    __syncthreads();
    const int ntn = (p.N + BNO - 1) / BNO;
    const int total = s_start[p.G] * ntn;
    const int logical = blockIdx.x;
    if (logical >= total) return;
    const int mt = logical / ntn;
    const int nt = logical - mt * ntn;
    int lo = 0, hi = p.G - 1;
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
    const float *W0 = shared ? p.Ws0 : p.W0 + g * wstride;
    const float *W1 = GATED ? (shared ? p.Ws1 : p.W1 + g * wstride) : nullptr;
    const float *bias = EPI == EPI_SWIGLU ? nullptr
                        : shared         ? p.bs
                        : (p.bias ? p.bias + (int64_t)g * N : nullptr);

    // loader mapping: one float4 of A per thread; one or two of B
    const int lrow = tid >> 2;       // 0..63
    const int lk = (tid & 3) * 4;    // 0,4,8,12
    const int64_t alr = m0 + lrow;
    const bool a_ok = alr < M;
    int64_t asrc = 0;
    if (a_ok) asrc = GATHER ? (shared ? alr : (int64_t)p.sorted_token[grow0 + alr]) : crow0 + alr;
    const float *a_ptr = p.A + asrc * K;
    const float *b_ptr[2];
    bool b_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int n = n0 + lrow;
        b_ok[h] = n < N && (h == 0 || GATED);
        const float *Wb = h == 0 ? W0 : W1;
        b_ptr[h] = b_ok[h] ? Wb + (int64_t)n * K : W0;
    }

    const int ty = tid >> 4, tx = tid & 15;
    float acc[4][4] = {}, accl[4][4] = {};
    for (int k0 = 0; k0 < K; k0 += BK) {
        const bool kok = k0 + lk < K;  // K is a multiple of 4
        float4 av = (a_ok && kok) ? *reinterpret_cast<const float4 *>(a_ptr + k0 + lk)
                                  : make_float4(0.f, 0.f, 0.f, 0.f);
        As[lk + 0][lrow] = av.x; As[lk + 1][lrow] = av.y;
        As[lk + 2][lrow] = av.z; As[lk + 3][lrow] = av.w;
#pragma unroll
        for (int h = 0; h < (GATED ? 2 : 1); ++h) {
            float4 bv = (b_ok[h] && kok) ? *reinterpret_cast<const float4 *>(b_ptr[h] + k0 + lk)
                                         : make_float4(0.f, 0.f, 0.f, 0.f);
            const int c = h * BNO + lrow;
            Bs[lk + 0][c] = bv.x; Bs[lk + 1][c] = bv.y;
            Bs[lk + 2][c] = bv.z; Bs[lk + 3][c] = bv.w;
        }
        __syncthreads();
#pragma unroll
        for (int kk = 0; kk < BK; ++kk) {
            float a[4], b[4], bl[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) a[i] = As[kk][ty * 4 + i];
#pragma unroll
            for (int j = 0; j < 4; ++j) b[j] = Bs[kk][tx * 4 + j];
            if (GATED) {
#pragma unroll
                for (int j = 0; j < 4; ++j) bl[j] = Bs[kk][BNO + tx * 4 + j];
            }
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    acc[i][j] = fmaf(a[i], b[j], acc[i][j]);
                    if (GATED) accl[i][j] = fmaf(a[i], bl[j], accl[i][j]);
                }
        }
        __syncthreads();
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t lr = m0 + ty * 4 + i;
        if (lr >= M) continue;
        float *crow = p.C + (crow0 + lr) * N;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int n = n0 + tx * 4 + j;
            if (n >= N) continue;
            float v;
            if (GATED) v = silu_exact(acc[i][j]) * accl[i][j];
            else {
                v = acc[i][j] + (bias ? bias[n] : 0.f);
                if (EPI == EPI_SILU_BIAS) v = silu_exact(v);
                if (EPI == EPI_GELU_BIAS) v = gelu_exact(v);
            }
            crow[n] = v;
        }
    }
}

template <int EPI, bool GATHER>
hipError_t launch_one(const GemmParamsF32 &p, int64_t max_mtiles, hipStream_t s) {
    const int64_t blocks = max_mtiles * ceil_div(p.N, 64);
    if (blocks == 0) return hipSuccess;
    grouped_gemm_f32_kernel<EPI, GATHER><<<(unsigned)blocks, 256, 0, s>>>(p);
    return hipGetLastError();
}

}  // namespace

hipError_t launch_grouped_ffn_f32(const moe_desc &d, const moe_weights &wt, const Workspace &w,
                                  const ExpertArgs &a, hipStream_t s, bool schedule_ready) {
    const bool glu = d.expert_kind == MOE_EXPERT_SWIGLU;
    int32_t *mtile_start = reinterpret_cast<int32_t *>(a.ws + w.mtile_start);
    constexpr int bm = kGemmBMf32;
    hipError_t e0 = schedule_ready ? hipSuccess : launch_schedule(d, a.offsets, mtile_start, bm, s);
    if (e0 != hipSuccess) return e0;
    // upper bound of the M tiles: sum_g ceil(rows_g / bm) <= ceil(R / bm) + E
    const int64_t max_mtiles = ceil_div(w.rows_routed_max, bm) +
                               std::min<int64_t>(d.E, w.rows_routed_max) +
                               (d.n_shared ? ceil_div(d.T, bm) : 0);
    float *H = reinterpret_cast<float *>(a.ws + w.H);
    GemmParamsF32 up{};
    up.A = (const float *)a.x;
    up.sorted_token = a.sorted_token;
    up.offsets = a.offsets;
    up.mtile_start = mtile_start;
    up.W0 = (const float *)wt.w_act;
    up.W1 = (const float *)wt.w_lin;
    up.bias = (const float *)wt.b_act;
    up.Ws0 = (const float *)wt.ws_act;
    up.Ws1 = (const float *)wt.ws_lin;
    up.bs = (const float *)wt.bs_act;
    up.C = H;
    up.T = d.T;
    up.shared_row0 = w.rows_routed_max;
    up.E = d.E;
    up.G = d.E + d.n_shared;
    up.N = d.d_ff;
    up.K = d.d_model;
    hipError_t e = glu ? launch_one<EPI_SWIGLU, true>(up, max_mtiles, s)
                   : d.expert_kind == MOE_EXPERT_GELU_MLP ? launch_one<EPI_GELU_BIAS, true>(up, max_mtiles, s)
                                                          : launch_one<EPI_SILU_BIAS, true>(up, max_mtiles, s);
    if (e != hipSuccess) return e;
    GemmParamsF32 dn = up;
    dn.A = H;
    dn.W0 = (const float *)wt.w_down;
    dn.W1 = nullptr;
    dn.bias = (const float *)wt.b_down;
    dn.Ws0 = (const float *)wt.ws_down;
    dn.Ws1 = nullptr;
    dn.bs = (const float *)wt.bs_down;
    dn.C = (float *)a.Y;
    dn.N = d.d_model;
    dn.K = d.d_ff;
    return launch_one<EPI_BIAS, false>(dn, max_mtiles, s);
}

}  // namespace moe
