// k_ternarize.hip -- absmean weight scale, ternary codes and 2-bit packing.
//
// "BitNet" quantization guide (Transformers docs, Portuguese), steps 1-2 of
// the numbered list, and "Transformers 实战 BitNet 1.58 位量化", section
// "BitLinear 的三步量化" steps 1-2: the scale of a weight tensor is its mean
// absolute value (one scale per tensor, floored at 1e-5); codes are the
// weights divided by it, rounded and clipped to {-1, 0, 1}.  Section
// "推理侧 BitLinear：打包权重、解包与缩放": codes + 1 take 2 bits each, four to
// a byte, so the packed tensor has a quarter of the rows.  Field i of packed
// row r holds weight row i*N/4 + r (plane order).
//
// Scale: two deterministic passes.  Pass 1 sums |W| in fp64 per workgroup
// over a fixed grid-stride pattern; pass 2 adds the partials in a fixed tree
// order, divides by the count, rounds to fp32 and applies the floor.
//
// Codes: division-free.  For fp32 w and m = w_mean, round_half_even(fl(w/m))
// is 0 exactly when |w|/m <= 1/2 + 2^-25 (the fp32 quotient rounds to at most
// 0.5 there, and 0.5 rounds to the even 0); elsewhere the rounded quotient is
// at least 1 in magnitude and clips to sign(w).  The product m*(1/2 + 2^-25)
// has at most 49 significant bits, so the fp64 comparison is exact.
#include "bl_common.h"

namespace bl {

namespace {

constexpr int kThreads = 256;

__device__ __forceinline__ double block_sum_fixed(double v, double *red) {
    v = wave_sum(v);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

template <bool VEC>
__global__ __launch_bounds__(kThreads) void k_absmean_partial(const float *__restrict__ W,
                                                              int64_t count,
                                                              double *__restrict__ partials) {
    __shared__ double red[4];
    double s = 0.0;
    const int64_t tid = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    const int64_t stride = (int64_t)gridDim.x * kThreads;
    if (VEC) {
        const int64_t n4 = count / 4;
        const float4 *W4 = reinterpret_cast<const float4 *>(W);
        for (int64_t i = tid; i < n4; i += stride) {
            float4 v = W4[i];
            s += fabs((double)v.x) + fabs((double)v.y) + fabs((double)v.z) + fabs((double)v.w);
        }
    } else {
        for (int64_t i = tid; i < count; i += stride) s += fabs((double)W[i]);
    }
    s = block_sum_fixed(s, red);
    if (threadIdx.x == 0) partials[blockIdx.x] = s;
}

__global__ __launch_bounds__(kThreads) void k_absmean_final(const double *__restrict__ partials,
                                                            int nparts, int64_t count,
                                                            float *__restrict__ w_mean) {
    __shared__ double red[4];
    double s = 0.0;
    for (int i = threadIdx.x; i < nparts; i += kThreads) s += partials[i];
    s = block_sum_fixed(s, red);
    if (threadIdx.x == 0) {
        float m = (float)(s / (double)count);
        w_mean[0] = m < 1e-5f ? 1e-5f : m;
    }
}

__device__ __forceinline__ uint32_t code_plus_one(float w, double thr) {
    // 0 -> code -1, 1 -> code 0, 2 -> code +1
    return fabs((double)w) <= thr ? 1u : (w > 0.0f ? 2u : 0u);
}

// One lane per 4 consecutive k of one packed row (K % 4 == 0).
__global__ __launch_bounds__(kThreads) void k_ternarize_pack4(const float *__restrict__ W, int N,
                                                              int K, const float *__restrict__ w_mean,
                                                              uint8_t *__restrict__ packed) {
    const int R = N / 4;
    const int K4 = K / 4;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (int64_t)R * K4) return;
    const int r = (int)(idx / K4);
    const int k = (int)(idx % K4) * 4;
    const double thr = (double)w_mean[0] * (0.5 + 0x1p-25);
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float4 v = *reinterpret_cast<const float4 *>(W + (int64_t)(i * R + r) * K + k);
        out |= code_plus_one(v.x, thr) << (2 * i);
        out |= code_plus_one(v.y, thr) << (8 + 2 * i);
        out |= code_plus_one(v.z, thr) << (16 + 2 * i);
        out |= code_plus_one(v.w, thr) << (24 + 2 * i);
    }
    *reinterpret_cast<uint32_t *>(packed + (int64_t)r * K + k) = out;
}

// One lane per packed byte (any K).
__global__ __launch_bounds__(kThreads) void k_ternarize_pack1(const float *__restrict__ W, int N,
                                                              int K, const float *__restrict__ w_mean,
                                                              uint8_t *__restrict__ packed) {
    const int R = N / 4;
    const int64_t idx = (int64_t)blockIdx.x * kThreads + threadIdx.x;
    if (idx >= (int64_t)R * K) return;
    const int r = (int)(idx / K);
    const int k = (int)(idx % K);
    const double thr = (double)w_mean[0] * (0.5 + 0x1p-25);
    uint32_t b = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) b |= code_plus_one(W[(int64_t)(i * R + r) * K + k], thr) << (2 * i);
    packed[idx] = (uint8_t)b;
}

} // namespace

int absmean_parts(int64_t count) {
    int64_t p = (count + kThreads * 64 - 1) / (kThreads * 64);
    if (p < 1) p = 1;
    if (p > 2048) p = 2048;
    return (int)p;
}

hipError_t launch_absmean(const float *W, int64_t count, double *partials, int nparts,
                          float *w_mean, hipStream_t s) {
    const bool vec = (count % 4 == 0) && ((uintptr_t)W % 16 == 0);
    if (vec)
        hipLaunchKernelGGL(k_absmean_partial<true>, dim3(nparts), dim3(kThreads), 0, s, W, count, partials);
    else
        hipLaunchKernelGGL(k_absmean_partial<false>, dim3(nparts), dim3(kThreads), 0, s, W, count, partials);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
    hipLaunchKernelGGL(k_absmean_final, dim3(1), dim3(kThreads), 0, s, partials, nparts, count, w_mean);
    return hipGetLastError();
}

hipError_t launch_ternarize_pack(const float *W, int N, int K, const float *w_mean, uint8_t *packed,
                                 hipStream_t s) {
    const int R = N / 4;
    if (K % 4 == 0 && (uintptr_t)W % 16 == 0 && (uintptr_t)packed % 4 == 0) {
        const int64_t n = (int64_t)R * (K / 4);
        hipLaunchKernelGGL(k_ternarize_pack4, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                           W, N, K, w_mean, packed);
    } else {
        const int64_t n = (int64_t)R * K;
        hipLaunchKernelGGL(k_ternarize_pack1, dim3((unsigned)((n + kThreads - 1) / kThreads)), dim3(kThreads), 0, s,
                           W, N, K, w_mean, packed);
    }
    return hipGetLastError();
}

} // namespace bl
