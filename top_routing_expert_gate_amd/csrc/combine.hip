// K4: weighted combine + shared-expert add for gfx950.
//
// out[t] = sum over kept slots s of w[t][s] * Y[row_of[t][s]] (+ Y_shared[t])
// (MoE-router build guide, step 5 combine; LLMs-from-scratch MoE guide,
// "Weighted aggregation"; DeepSeek 5.7, section 4).  Dropped slots
// (row_of < 0) add nothing.  A gather, not a scatter: each thread owns one
// 16-byte chunk of one output row and reads the k source rows' matching
// chunks, so every load and store is a coalesced 16-byte access, there are
// no atomics, and the f32 sum runs in slot order with the shared row last --
// bit-for-bit reproducible.
#include "moe_internal.h"

namespace moe {
namespace {

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
};

template <typename T>
__global__ __launch_bounds__(256) void combine_kernel(const T *__restrict__ Y,
                                                      const T *__restrict__ Ys,
                                                      const int32_t *__restrict__ row_of,
                                                      const float *__restrict__ w,
                                                      T *__restrict__ out, int64_t ntok, int d,
                                                      int k) {
    constexpr int N = Chunk<T>::n;
    const int cpr = d / N;  // chunks per row
    const int64_t total = ntok * cpr;
    for (int64_t g = (int64_t)blockIdx.x * blockDim.x + threadIdx.x; g < total;
         g += (int64_t)gridDim.x * blockDim.x) {
        const int64_t t = g / cpr;
        const int c = (int)(g - t * cpr);
        float acc[N];
#pragma unroll
        for (int i = 0; i < N; ++i) acc[i] = 0.f;
        for (int s = 0; s < k; ++s) {
            const int r = row_of[t * k + s];
            if (r < 0) continue;
            const float ws = w[t * k + s];
            float v[N];
            Chunk<T>::load(Y + (int64_t)r * d + (int64_t)c * N, v);
#pragma unroll
            for (int i = 0; i < N; ++i) acc[i] = fmaf(ws, v[i], acc[i]);
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

hipError_t launch_combine(const moe_desc &d, const void *Y, const void *Y_shared,
                          const int32_t *row_of, const float *topk_w, void *out,
                          hipStream_t s) {
    const int n = d.dtype == MOE_BF16 ? 8 : 4;
    const int64_t total = d.T * (d.d_model / n);
    // enough workgroups to fill 256 CUs several times over; grid-stride beyond
    const unsigned blocks = (unsigned)std::min<int64_t>(ceil_div(total, 256), 256 * 32);
    if (d.dtype == MOE_BF16)
        combine_kernel<__bf16><<<blocks, 256, 0, s>>>((const __bf16 *)Y, (const __bf16 *)Y_shared,
                                                      row_of, topk_w, (__bf16 *)out, d.T,
                                                      d.d_model, d.k);
    else
        combine_kernel<float><<<blocks, 256, 0, s>>>((const float *)Y, (const float *)Y_shared,
                                                     row_of, topk_w, (float *)out, d.T,
                                                     d.d_model, d.k);
    return hipGetLastError();
}

}  // namespace moe
