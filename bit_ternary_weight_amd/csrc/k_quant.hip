// k_quant.hip -- per-token activation quantization, and RMSNorm fused with it.
//
// Activation quantization: "BitNet" quantization guide (Transformers docs,
// Portuguese), step 3 of the numbered list; "Transformers 实战 BitNet 1.58 位量化",
// section "BitLinear 的三步量化", step 3: every token row is scaled by
// 127 / max|x| (the max floored at 1e-5), rounded, and clipped to [-128, 127].
// RMSNorm (subln / ffn_sub_norm): the subln paragraph after "推理侧 BitLinear"
// on the same page, with rms_norm_eps from "BitNetConfig" on the BitNet model
// documentation pages.
//
// One workgroup (256 lanes = 4 waves) per token row.  Rows are short
// (<= 6912 elements), so the second and third passes re-read the row from
// L2 instead of holding it in registers.  The row maximum is exact in any
// order; the fp64 sum of squares is reduced in a fixed tree order.
#include "bl_common.h"

namespace bl {

namespace {

constexpr int kThreads = 256;
constexpr float kFloor = 1e-5f;

template <typename T>
__device__ __forceinline__ float load_elem(const T *p, int64_t i);
template <>
__device__ __forceinline__ float load_elem<float>(const float *p, int64_t i) { return p[i]; }
template <>
__device__ __forceinline__ float load_elem<uint16_t>(const uint16_t *p, int64_t i) {
    return bf16_to_f32(p[i]);
}

// Loads 4 consecutive elements starting at i (i % 4 == 0 and the row base is
// 8-byte aligned for bf16 / 16-byte aligned for fp32).
template <typename T>
__device__ __forceinline__ void load4(const T *p, int64_t i, float v[4]);
template <>
__device__ __forceinline__ void load4<float>(const float *p, int64_t i, float v[4]) {
    float4 t = *reinterpret_cast<const float4 *>(p + i);
    v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
}
template <>
__device__ __forceinline__ void load4<uint16_t>(const uint16_t *p, int64_t i, float v[4]) {
    uint2 t = *reinterpret_cast<const uint2 *>(p + i);
    v[0] = __uint_as_float(t.x << 16);
    v[1] = __uint_as_float(t.x & 0xFFFF0000u);
    v[2] = __uint_as_float(t.y << 16);
    v[3] = __uint_as_float(t.y & 0xFFFF0000u);
}

__device__ __forceinline__ int quant1(float v, float a) {
    float r = rintf(v * a);            // fp32 product, round half to even
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

__device__ __forceinline__ uint32_t pack4(int c0, int c1, int c2, int c3) {
    return (uint32_t)(c0 & 0xFF) | ((uint32_t)(c1 & 0xFF) << 8) | ((uint32_t)(c2 & 0xFF) << 16) |
           ((uint32_t)(c3 & 0xFF) << 24);
}

__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

__device__ __forceinline__ double block_sum(double v, double *red) {
    v = wave_sum(v);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    __syncthreads();
    double r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

// Value of element k of the row after the optional RMSNorm (r, g); with
// NORM == false it is the raw element.
template <typename T, bool NORM>
__device__ __forceinline__ float elem(const T *row, int64_t k, float r, const float *g) {
    float v = load_elem<T>(row, k);
    if (NORM) {
        v = v * r;
        if (g) v = v * g[k];
    }
    return v;
}

template <typename T, bool NORM, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const T *__restrict__ x, int K, int ldx,
                                                         const float *__restrict__ g, float eps,
                                                         int8_t *__restrict__ q,
                                                         float *__restrict__ a) {
    __shared__ float redf[4];
    __shared__ double redd[4];
    const int m = blockIdx.x;
    const T *row = x + (int64_t)m * ldx;
    int8_t *qrow = q + (int64_t)m * K;

    float r = 1.0f;
    if (NORM) {
        double ss = 0.0;
        if (VEC) {
            for (int k = threadIdx.x * 4; k < K; k += kThreads * 4) {
                float v[4];
                load4<T>(row, k, v);
#pragma unroll
                for (int i = 0; i < 4; ++i) ss += (double)v[i] * (double)v[i];
            }
        } else {
            for (int k = threadIdx.x; k < K; k += kThreads) {
                double v = (double)load_elem<T>(row, k);
                ss += v * v;
            }
        }
        ss = block_sum(ss, redd);
        r = (float)(1.0 / sqrt(ss / (double)K + (double)eps));
    }

    float amax = 0.0f;
    if (VEC) {
        for (int k = threadIdx.x * 4; k < K; k += kThreads * 4) {
            float v[4];
            load4<T>(row, k, v);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t = v[i];
                if (NORM) {
                    t = t * r;
                    if (g) t = t * g[k + i];
                }
                amax = fmaxf(amax, fabsf(t));
            }
        }
    } else {
        for (int k = threadIdx.x; k < K; k += kThreads)
            amax = fmaxf(amax, fabsf(elem<T, NORM>(row, k, r, g)));
    }
    amax = block_max(amax, redf);
    const float s = 127.0f / fmaxf(amax, kFloor);   // IEEE fp32 division
    if (threadIdx.x == 0) a[m] = s;

    if (VEC) {
        for (int k = threadIdx.x * 4; k < K; k += kThreads * 4) {
            float v[4];
            load4<T>(row, k, v);
            int c[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                float t = v[i];
                if (NORM) {
                    t = t * r;
                    if (g) t = t * g[k + i];
                }
                c[i] = quant1(t, s);
            }
            *reinterpret_cast<uint32_t *>(qrow + k) = pack4(c[0], c[1], c[2], c[3]);
        }
    } else {
        for (int k = threadIdx.x; k < K; k += kThreads)
            qrow[k] = (int8_t)quant1(elem<T, NORM>(row, k, r, g), s);
    }
}

template <bool NORM>
hipError_t launch_rows(const void *x, int dt, int M, int K, int ldx, const float *g, float eps,
                       int8_t *q, float *a, hipStream_t s) {
    // Vector path: 4 elements per access, every row start aligned for it.
    const int esz = dt == BL_BF16 ? 2 : 4;
    const bool vec = (K % 4 == 0) && (ldx % 4 == 0) && ((uintptr_t)x % (4 * esz) == 0) &&
                     ((uintptr_t)q % 4 == 0);
    dim3 grid(M), block(kThreads);
    if (dt == BL_BF16) {
        const uint16_t *xp = (const uint16_t *)x;
        if (vec)
            hipLaunchKernelGGL((k_quant_rows<uint16_t, NORM, true>), grid, block, 0, s, xp, K, ldx, g, eps, q, a);
        else
            hipLaunchKernelGGL((k_quant_rows<uint16_t, NORM, false>), grid, block, 0, s, xp, K, ldx, g, eps, q, a);
    } else {
        const float *xp = (const float *)x;
        if (vec)
            hipLaunchKernelGGL((k_quant_rows<float, NORM, true>), grid, block, 0, s, xp, K, ldx, g, eps, q, a);
        else
            hipLaunchKernelGGL((k_quant_rows<float, NORM, false>), grid, block, 0, s, xp, K, ldx, g, eps, q, a);
    }
    return hipGetLastError();
}

// Several independent quantizations in one launch: block b quantizes row
// b - row0 of the problem whose [row0, row0 + M) range holds b.
__global__ __launch_bounds__(kThreads) void k_quant_batch(QuantBatch qb) {
    __shared__ float redf[4];
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < qb.n && (int)blockIdx.x >= qb.p[i].row0) pi = i;
    const QuantProblem &p = qb.p[pi];
    const int m = (int)blockIdx.x - p.row0;
    const int K = p.K;
    float amax = 0.0f;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const size_t i = (size_t)m * p.ldx + k;
        const float v = p.x_dt == BL_BF16 ? bf16_to_f32(((const uint16_t *)p.x)[i]) : ((const float *)p.x)[i];
        amax = fmaxf(amax, fabsf(v));
    }
    amax = block_max(amax, redf);
    const float s = 127.0f / fmaxf(amax, kFloor);
    if (threadIdx.x == 0) p.a[m] = s;
    for (int k = threadIdx.x; k < K; k += kThreads) {
        const size_t i = (size_t)m * p.ldx + k;
        const float v = p.x_dt == BL_BF16 ? bf16_to_f32(((const uint16_t *)p.x)[i]) : ((const float *)p.x)[i];
        p.q[(size_t)m * K + k] = (int8_t)quant1(v, s);
    }
}

} // namespace

hipError_t launch_quant_batch(QuantBatch &qb, hipStream_t s) {
    int rows = 0;
    for (int i = 0; i < qb.n; ++i) {
        qb.p[i].row0 = rows;
        rows += qb.p[i].M;
    }
    if (rows == 0) return hipSuccess;
    hipLaunchKernelGGL(k_quant_batch, dim3(rows), dim3(kThreads), 0, s, qb);
    return hipGetLastError();
}

hipError_t launch_quant_act(const void *x, int x_dt, int M, int K, int ldx, int8_t *q, float *a,
                            hipStream_t s) {
    return launch_rows<false>(x, x_dt, M, K, ldx, nullptr, 0.0f, q, a, s);
}

hipError_t launch_rmsnorm_quant(const void *h, int h_dt, int M, int K, const float *g, float eps,
                                int8_t *q, float *a, hipStream_t s) {
    return launch_rows<true>(h, h_dt, M, K, K, g, eps, q, a, s);
}

} // namespace bl
