// K4: weighted combine + shared-expert add for gfx950.
//
// out[t] = sum over kept slots s of w[t][s] * Y[row_of[t][s]] (+ Y_shared[t])
// (MoE-router build guide, step 5 combine; LLMs-from-scratch MoE guide,
// "Weighted aggregation"; DeepSeek 5.7, section 4).  Dropped slots
// (row_of < 0) add nothing, or with the residual drop policy w * x[t] (Expert
// Networks, In[10]: a dropped token passes through).  A gather, not a scatter: each thread owns one
// 16-byte chunk of one output row and reads the k source rows' matching
// chunks, so every load and store is a coalesced 16-byte access, there are
// no atomics, and the f32 sum runs in slot order with the shared row last --
// bit-for-bit reproducible.  Y is addressed through row_of, which for the
// moe_combine entry point may point anywhere in a caller buffer of at most
// min(T*k, E*capacity) rows; rows are addressed with 64-bit arithmetic, so
// that buffer may exceed 2 GiB.
#include "moe_internal.h"

namespace moe {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

template <typename T>
struct Chunk;
template <>
struct Chunk<float> {
    static constexpr int n = 4;
    typedef float4 vec;
    __device__ static void load(const float *p, float *v) {
        float4 q = *reinterpret_cast<const float4 *>(p);
        v[0] = q.x; v[1] = q.y; v[2] = q.z; v[3] = q.w;
    }
    __device__ static void store(float *p, const float *v) {
        *reinterpret_cast<float4 *>(p) = make_float4(v[0], v[1], v[2], v[3]);
    }
    __device__ static void unpack(u32x4 q, float *v) {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float(q[i]);
    }
};
template <>
struct Chunk<__bf16> {
    static constexpr int n = 8;
    typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
    __device__ static void load(const __bf16 *p, float *v) {
        bf16x8 q = *reinterpret_cast<const bf16x8 *>(p);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)q[i];
    }
    __device__ static void store(__bf16 *p, const float *v) {
        bf16x8 q;
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = (__bf16)v[i];
        *reinterpret_cast<bf16x8 *>(p) = q;
    }
    __device__ static void unpack(u32x4 q, float *v) {
        bf16x8 b = __builtin_bit_cast(bf16x8, q);
#pragma unroll
        for (int i = 0; i < 8; ++i) v[i] = (float)b[i];
    }
};

// KMAX = k rounded up to 1, 2, 4 or 8 (0: any k, slots walked in a loop).
// With KMAX > 0 all source rows of a chunk are requested before the first
// multiply, so the k gathers overlap instead of running one after another;
// dropped slots (row_of < 0) read zeros through an out-of-range buffer offset.
// RESID: a dropped slot reads the token's own row of X instead (and a kept
// slot reads zeros from X the same way).
// WAVE_TOKEN: the chunks per row are a multiple of 64, so every wavefront
// works on one token; its slot indices and weights are then read once per
// wavefront through the scalar cache instead of once per lane.
template <typename T, int KMAX, bool RESID, bool WAVE_TOKEN>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ Y,
                                                      const T *__restrict__ Ys,
                                                      const T *__restrict__ X,
                                                      const int32_t *__restrict__ row_of,
                                                      const float *__restrict__ w,
                                                      T *__restrict__ out, int64_t ntok, int d,
                                                      int k, int x_bytes) {
    constexpr int N = Chunk<T>::n;
    const int cpr = d / N;  // chunks per row
    const int64_t total = ntok * cpr;
    const u32x4 zero = {0u, 0u, 0u, 0u};
    const __amdgpu_buffer_rsrc_t rX = __builtin_amdgcn_make_buffer_rsrc(
        const_cast<T *>(RESID ? X : Y), (short)0, RESID ? x_bytes : 0, 0x00020000);
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = WAVE_TOKEN ? (int64_t)__builtin_amdgcn_readfirstlane((int)(g / cpr)) : g / cpr;
        const int c = (int)(g - t * cpr);
        float acc[N];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = 0.f;
        if (KMAX > 0) {
            u32x4 raw[KMAX > 0 ? KMAX : 1];
            float ws[KMAX > 0 ? KMAX : 1];
            const int xoff = (int)((t * d + (int64_t)c * N) * sizeof(T));
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                const int r = s < k ? row_of[t * k + s] : -1;
                ws[s] = s < k ? w[t * k + s] : 0.f;
                if (WAVE_TOKEN) {
                    // the slot's row is the same for the whole wavefront: a
                    // descriptor over that row alone (empty for a dropped
                    // slot, which then reads zeros), so Y may exceed the
                    // 2 GiB a 32-bit offset reaches
                    const int ru = __builtin_amdgcn_readfirstlane(r);
                    const __amdgpu_buffer_rsrc_t rY = __builtin_amdgcn_make_buffer_rsrc(
                        const_cast<T *>(Y + (int64_t)(ru >= 0 ? ru : 0) * d), (short)0,
                        ru >= 0 ? d * (int)sizeof(T) : 0, 0x00020000);
                    raw[s] = __builtin_amdgcn_raw_buffer_load_b128(rY, c * N * (int)sizeof(T), 0, 0);
                } else {
                    raw[s] = r >= 0 ? *reinterpret_cast<const u32x4 *>(Y + (int64_t)r * d + (int64_t)c * N)
                                    : zero;
                }
                if (RESID) {
                    const u32x4 xr = __builtin_amdgcn_raw_buffer_load_b128(
                        rX, r < 0 && s < k ? xoff : (int)0x80000000u, 0, 0);
                    raw[s] |= xr;  // one of the two reads is zeros
                }
            }
#pragma unroll
            for (int s = 0; s < KMAX; ++s) {
                float v[N];
                Chunk<T>::unpack(raw[s], v);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[i] = fmaf(ws[s], v[i], acc[i]);
            }
        } else {
            for (int s = 0; s < k; ++s) {
                const int r = row_of[t * k + s];
                if (r < 0 && !RESID) continue;
                const float ws = w[t * k + s];
                float v[N];
                Chunk<T>::load(r >= 0 ? Y + (int64_t)r * d + (int64_t)c * N : X + t * d + (int64_t)c * N, v);
#pragma unroll
                for (int i = 0; i < N; ++i) acc[i] = fmaf(ws, v[i], acc[i]);
            }
        }
        if (Ys) {
            float v[N];
            Chunk<T>::load(Ys + t * d + (int64_t)c * N, v);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] += v[i];
        }
        Chunk<T>::store(out + t * d + (int64_t)c * N, acc);
    }
}

}  // namespace

hipError_t launch_combine(const moe_desc &d, const void *Y, const void *Y_shared, const void *x,
                          const int32_t *row_of, const float *topk_w, void *out,
                          hipStream_t s) {
    const int n = d.dtype == MOE_BF16 ? 8 : 4;
    const int64_t total = d.T * (d.d_model / n);
    // enough workgroups to fill 256 CUs several times over; grid-stride beyond
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(total, 256), 256 * 32);
    const int kmax = d.k <= 1 ? 1 : d.k <= 2 ? 2 : d.k <= 4 ? 4 : d.k <= 8 ? 8 : 0;
    const int x_bytes = (int)std::min<int64_t>(d.T * d.d_model * elem_bytes(d.dtype), INT32_MAX);
    const bool resid = d.drop_policy == MOE_DROP_RESIDUAL;
    const bool wave_token = (d.d_model / n) % 64 == 0;
#define MOE_COMBINE_RW(TY, KM, R, WT)                                                        \
    combine_kernel<TY, KM, R, WT><<<blocks, 256, 0, s>>>((const TY *)Y, (const TY *)Y_shared, \
                                                         (const TY *)x, row_of, topk_w, (TY *)out, \
                                                         d.T, d.d_model, d.k, x_bytes)
#define MOE_COMBINE_R(TY, KM, R)                                                             \
    do {                                                                                    \
        if (KM > 0 && wave_token) MOE_COMBINE_RW(TY, KM, R, true);                          \
        else MOE_COMBINE_RW(TY, KM, R, false);                                              \
    } while (0)
#define MOE_COMBINE(TY, KM)                                                                 \
    do {                                                                                    \
        if (resid) MOE_COMBINE_R(TY, KM, true);                                             \
        else MOE_COMBINE_R(TY, KM, false);                                                  \
    } while (0)
    if (d.dtype == MOE_BF16) {
        switch (kmax) {
            case 1: MOE_COMBINE(__bf16, 1); break;
            case 2: MOE_COMBINE(__bf16, 2); break;
            case 4: MOE_COMBINE(__bf16, 4); break;
            case 8: MOE_COMBINE(__bf16, 8); break;
            default: MOE_COMBINE(__bf16, 0); break;
        }
    } else {
        switch (kmax) {
            case 1: MOE_COMBINE(float, 1); break;
            case 2: MOE_COMBINE(float, 2); break;
            case 4: MOE_COMBINE(float, 4); break;
            case 8: MOE_COMBINE(float, 8); break;
            default: MOE_COMBINE(float, 0); break;
        }
    }
#undef MOE_COMBINE
#undef MOE_COMBINE_R
#undef MOE_COMBINE_RW
    return hipGetLastError();
}

}  // namespace moe
