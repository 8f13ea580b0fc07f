// bl_common.h -- internal declarations shared by the libbitlinear HIP sources.
// Not part of the public ABI (that is include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Packed-row layout of a (possibly segmented) packed weight.  Segment s owns
// packed rows [roff[s], roff[s+1]); its output columns start at 4*roff[s] and
// field f of its local packed row r is output column 4*roff[s] + f*R_s + r,
// with R_s = roff[s+1] - roff[s] (plane order).
struct SegTab {
    int n;
    int roff[BL_MAX_SEGMENTS + 1];
};

// Location of one output column: segment index and column.
struct ColOf {
    int seg;
    int col;
};

__device__ __forceinline__ ColOf col_of(const SegTab &t, int rr, int f) {
    int s = 0;
#pragma unroll
    for (int i = 1; i < BL_MAX_SEGMENTS; ++i)
        if (i < t.n && rr >= t.roff[i]) s = i;
    int r0 = t.roff[s];
    int Rs = t.roff[s + 1] - r0;
    return ColOf{s, 4 * r0 + f * Rs + (rr - r0)};
}

__device__ __forceinline__ float bf16_to_f32(uint16_t b) {
    return __uint_as_float(((uint32_t)b) << 16);
}

// fp32 -> bf16, round to nearest even (finite input).
__device__ __forceinline__ uint16_t f32_to_bf16(float v) {
    uint32_t u = __float_as_uint(v);
    u += 0x7FFFu + ((u >> 16) & 1u);
    return (uint16_t)(u >> 16);
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v = fmaxf(v, __shfl_xor(v, o, 64));
    return v;
}

__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) v += __shfl_xor(v, o, 64);
    return v;
}

// Output writer shared by the contraction kernels: A is the exact int32
// accumulator, scale = w_mean_s / a_m (already computed in fp32).
__device__ __forceinline__ void store_out(void *y, int y_dt, size_t idx, int A, float scale) {
    if (y_dt == BL_I32) {
        ((int32_t *)y)[idx] = A;
    } else {
        float v = (float)A * scale;
        if (y_dt == BL_F32)
            ((float *)y)[idx] = v;
        else
            ((uint16_t *)y)[idx] = f32_to_bf16(v);
    }
}

// ReLU^2(gate) * up on already-rescaled fp32 values (two roundings, no FMA).
__device__ __forceinline__ float relu2_mul(float g, float u) {
    float gp = g > 0.0f ? g : 0.0f;
    float sq = gp * gp;
    return sq * u;
}

// ---------------------------------------------------------------------------
// Launchers (host side).  Each returns hipSuccess or the launch error.
// ---------------------------------------------------------------------------
hipError_t launch_absmean(const float *W, int64_t count, double *partials, int nparts,
                          float *w_mean, hipStream_t s);
int absmean_parts(int64_t count);
hipError_t launch_ternarize_pack(const float *W, int N, int K, const float *w_mean,
                                 uint8_t *packed, hipStream_t s);

hipError_t launch_quant_act(const void *x, int x_dt, int M, int K, int ldx, int8_t *q, float *a,
                            hipStream_t s);
hipError_t launch_rmsnorm_quant(const void *h, int h_dt, int M, int K, const float *g, float eps,
                                int8_t *q, float *a, hipStream_t s);

// Contraction arguments common to the decode and prefill kernels.
struct Contract {
    const int8_t *q;  // [M,K] codes, row stride ldq
    int ldq;
    const float *a;   // [M] activation scales
    int M, K;
    const uint8_t *P; // packed weight, row stride K
    SegTab seg;       // packed-row layout (for PAIR: the gate tensor's rows only)
    int R;            // packed rows addressed (for PAIR: gate rows)
    const float *w_mean;
    void *y;          // [M, ldy]
    int y_dt;
    int ldy;
    bool pair;        // gate|up with ReLU^2(gate)*up epilogue; up rows at P + R*K
};

// Decode path (M <= 64).  acc/tickets: zero-initialised scratch, left zero.
hipError_t launch_gemv(const Contract &c, int32_t *acc, size_t acc_cap, unsigned *tickets,
                       int ticket_cap, hipStream_t s);
// Prefill path (any M).
hipError_t launch_gemm(const Contract &c, hipStream_t s);
// Any K (slow, simple): used when K is not a multiple of 16.
hipError_t launch_generic(const Contract &c, hipStream_t s);

} // namespace bl
