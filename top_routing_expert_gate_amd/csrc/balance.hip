// Balance statistics of a routing for gfx950.
//
// SNEPPX SER MoE tutorial, step 4 "Load-balancing loss": the loss is
// coef * sum_e frac_e * p_avg_e, where frac_e is the share of the tokens'
// top-k routes that went to expert e (routes / tokens) and p_avg_e is the mean
// over tokens of the softmax over all experts of the router logits.  DeepSeek
// 5.7, "Implementation and measurement plan", asks for a load histogram and a
// coefficient-of-variation diagnostic: the histogram is moe_dispatch's
// counts_assigned, the spread is computed here.
//
//   balance_partial  one workgroup per block of token rows; each wave takes
//                    rows in turn, one lane per expert (up to 4 per lane):
//                    row maximum and sum of exponentials by wave reductions,
//                    then every lane adds its probabilities to double
//                    accumulators; the four waves' sums are added in wave
//                    order into one partial row per workgroup
//   balance_final    one workgroup: partial rows summed in block order, the
//                    loss, and mean / deviation / maximum of the counts
//
// Every sum runs in a fixed order, so the statistics are bit-reproducible.
#include <math.h>

#include "moe_internal.h"

namespace moe {
namespace {

__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v = fmaxf(v, __shfl_xor(v, m));
    return v;
}

__device__ __forceinline__ float wave_sum_f32(float v) {
#pragma unroll
    for (int m = 32; m > 0; m >>= 1) v += __shfl_xor(v, m);
    return v;
}

constexpr int kBalWaves = 4;

__global__ __launch_bounds__(kBalWaves * 64) void balance_partial_kernel(
    const float *__restrict__ logits, int64_t T, int E, int rows_per_block,
    double *__restrict__ part) {
    __shared__ double red[kBalWaves][MOE_MAX_EXPERTS];
    const int lane = threadIdx.x & 63;
    const int wave = threadIdx.x >> 6;
    const int64_t r0 = (int64_t)blockIdx.x * rows_per_block;
    const int64_t r1 = min(T, r0 + rows_per_block);
    double acc[4] = {0.0, 0.0, 0.0, 0.0};
    for (int64_t row = r0 + wave; row < r1; row += kBalWaves) {
        const float *lr = logits + row * E;
        float l[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int e = lane + 64 * j;
            l[j] = e < E ? lr[e] : -INFINITY;
        }
        const float m = wave_max_f32(fmaxf(fmaxf(l[0], l[1]), fmaxf(l[2], l[3])));
        float ex[4], s = 0.f;
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            ex[j] = lane + 64 * j < E ? expf(l[j] - m) : 0.f;
            s += ex[j];
        }
        const float inv = 1.0f / wave_sum_f32(s);
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[j] += (double)(ex[j] * inv);
    }
#pragma unroll
    for (int j = 0; j < 4; ++j)
        if (lane + 64 * j < E) red[wave][lane + 64 * j] = acc[j];
    __syncthreads();
    for (int e = threadIdx.x; e < E; e += blockDim.x) {
        double v = 0.0;
#pragma unroll
        for (int w = 0; w < kBalWaves; ++w) v += red[w][e];
        part[(int64_t)blockIdx.x * E + e] = v;
    }
}

__global__ __launch_bounds__(256) void balance_final_kernel(
    const double *__restrict__ part, int nblk, const int32_t *__restrict__ counts, int64_t T,
    int E, float coef, float *__restrict__ p_mean, float *__restrict__ stats) {
    __shared__ double s_dot[256], s_cnt[256], s_sq[256];
    __shared__ double s_max[256];
    const int e = threadIdx.x;
    double dot = 0.0, c = 0.0;
    if (e < E) {
        double p = 0.0;
        for (int b = 0; b < nblk; ++b) p += part[(int64_t)b * E + e];
        p /= (double)T;
        if (p_mean) p_mean[e] = (float)p;
        c = (double)counts[e];
        dot = (c / (double)T) * p;
    }
    s_dot[e] = dot;
    s_cnt[e] = c;
    s_max[e] = e < E ? c : 0.0;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {  // fixed tree
        if (e < h) {
            s_dot[e] += s_dot[e + h];
            s_cnt[e] += s_cnt[e + h];
            s_max[e] = fmax(s_max[e], s_max[e + h]);
        }
        __syncthreads();
    }
    const double mean = s_cnt[0] / (double)E;
    const double dev = e < E ? (c - mean) : 0.0;
    s_sq[e] = dev * dev;
    __syncthreads();
    for (int h = 128; h > 0; h >>= 1) {
        if (e < h) s_sq[e] += s_sq[e + h];
        __syncthreads();
    }
    if (e == 0) {
        stats[0] = (float)((double)coef * s_dot[0]);
        stats[1] = (float)(sqrt(s_sq[0] / (double)E) / mean);
        stats[2] = (float)(s_max[0] / mean);
    }
}

}  // namespace

hipError_t launch_balance(const moe_desc &d, const Workspace &w, const float *logits,
                          const int32_t *counts_assigned, float coef, float *p_mean,
                          float *stats, char *ws, hipStream_t s) {
    double *part = reinterpret_cast<double *>(ws + w.balance);
    balance_partial_kernel<<<w.bal_blocks, kBalWaves * 64, 0, s>>>(logits, d.T, d.E, w.bal_rows,
                                                                    part);
    balance_final_kernel<<<1, 256, 0, s>>>(part, w.bal_blocks, counts_assigned, d.T, d.E, coef,
                                           p_mean, stats);
    return hipGetLastError();
}

}  // namespace moe
