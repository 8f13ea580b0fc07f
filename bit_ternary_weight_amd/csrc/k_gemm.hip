// k_gemm.hip -- prefill-path BitLinear (any M): int8 x ternary GEMM on the
// matrix cores, plus a plain kernel for K that is not a multiple of 16.
//
// "Transformers 实战 BitNet 1.58 位量化", section "推理侧 BitLinear：打包权重、解包与缩放":
// the inference forward multiplies the int8 activations with the unpacked
// ternary weight and rescales the product by the activation and weight
// scales; the unpack reads field i of a packed byte under the mask 3 << 2i
// and subtracts 1.  The weights are never unpacked to memory: the 2-bit
// fields are expanded in registers (see the helpers in bl_common.h).
#include "bl_common.h"

namespace bl {

namespace {

// Final output of one accumulator entry of a Contract.
__device__ __forceinline__ void emit(const Contract &c, int m, int vr, int f, int A, int U) {
    emit_out(c.y, c.y_dt, c.ldy, c.pair, c.seg, c.R, c.w_mean, m, vr, f, c.a[m], A, U);
}

// ===========================================================================
// Prefill kernel (any M).
// Workgroup tile: 128 token rows x 32 packed rows (= 128 output columns; PAIR:
// 32 gate rows + 32 up rows), 4 waves in a 2 x 2 grid, 64-wide k-steps.
// Global -> registers -> LDS, double buffered: the next step's tile is in
// flight while the matrix cores work on the current one.  LDS holds each
// 16-row x 64-k piece in "fragment order" (lane l's 16 bytes at 16*l), so the
// LDS writes and the operand reads are both linear.  Each wave expands its
// 16 packed rows into the four field operands in registers.
// ===========================================================================
constexpr int kBM = 128;
constexpr int kVR = 32;

template <bool PAIR>
__global__ __launch_bounds__(256) void k_gemm(Contract c, int ntm) {
    constexpr int BR = PAIR ? 2 * kVR : kVR;      // packed rows staged per step
    constexpr int NBF = BR / 16;                   // 16-row B pieces per step
    constexpr int NB = PAIR ? 2 : 1;
    __shared__ __attribute__((aligned(16))) int8_t sA[2][kBM * 64];
    __shared__ __attribute__((aligned(16))) uint8_t sB[2][BR * 64];

    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int g = lane >> 4;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int bm = blockIdx.x % ntm;
    const int bn = blockIdx.x / ntm;
    const int m0 = bm * kBM;
    const int r0 = bn * kVR;
    const int K = c.K;
    const int nsteps = (K + 63) >> 6;

    // Loader assignments (fixed per thread).
    // A: pieces cid = tid and tid + 256 of 512 (8 row groups x 64 lanes).
    const int8_t *ga[2];
    bool a_ok[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int cid = tid + 256 * h;
        const int row = (cid >> 6) * 16 + (cid & 15);
        const int gg = (cid >> 4) & 3;
        a_ok[h] = (m0 + row) < c.M;
        ga[h] = c.q + (size_t)(a_ok[h] ? m0 + row : 0) * c.ldq + 16 * gg;
    }
    // B: piece cid = tid when tid < BR*4.
    const bool b_loader = tid < BR * 4;
    const uint8_t *gb;
    bool b_ok;
    {
        const int cid = tid;
        const int fr = cid >> 6;
        const int gg = (cid >> 4) & 3;
        int vrow = r0 + (fr % (kVR / 16)) * 16 + (cid & 15);
        b_ok = b_loader && vrow < c.R;
        const int prow = (PAIR && fr >= kVR / 16) ? c.R + vrow : vrow;
        gb = c.P + (size_t)(b_ok ? prow : 0) * K + 16 * gg;
    }
    const int a_kg[2] = {16 * ((tid >> 4) & 3), 16 * (((tid + 256) >> 4) & 3)};
    const int b_kg = 16 * ((tid >> 4) & 3);

    v4i ra[2], rb;
    auto gload = [&](int st) {
        const int k0 = st * 64;
#pragma unroll
        for (int h = 0; h < 2; ++h)
            ra[h] = (a_ok[h] && k0 + a_kg[h] < K) ? ld16(ga[h] + k0) : v4i{0, 0, 0, 0};
        rb = (b_ok && k0 + b_kg < K) ? ld16(gb + k0) : v4i{0, 0, 0, 0};
    };
    auto lstore = [&](int buf) {
#pragma unroll
        for (int h = 0; h < 2; ++h)
            *reinterpret_cast<v4i *>(&sA[buf][(tid + 256 * h) * 16]) = ra[h];
        if (b_loader) *reinterpret_cast<v4i *>(&sB[buf][tid * 16]) = rb;
    };

    v4i accv[NB][4][4];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int i = 0; i < 4; ++i)
#pragma unroll
            for (int f = 0; f < 4; ++f) accv[t][i][f] = v4i{0, 0, 0, 0};
    int qs[4] = {0, 0, 0, 0};

    gload(0);
    lstore(0);
    __syncthreads();

    for (int st = 0; st < nsteps; ++st) {
        const int buf = st & 1;
        if (st + 1 < nsteps) gload(st + 1);
        v4i af[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
            af[i] = *reinterpret_cast<const v4i *>(&sA[buf][((wm * 4 + i) * 64 + lane) * 16]);
#pragma unroll
        for (int i = 0; i < 4; ++i) qs[i] += rowsum16(af[i]);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            const int fr = t * (kVR / 16) + wn;
            const v4i b = *reinterpret_cast<const v4i *>(&sB[buf][(fr * 64 + lane) * 16]);
            v4i fb[4];
            expand(b, fb);
#pragma unroll
            for (int i = 0; i < 4; ++i)
#pragma unroll
                for (int f = 0; f < 4; ++f) accv[t][i][f] = mfma16(af[i], fb[f], accv[t][i][f]);
        }
        if (st + 1 < nsteps) lstore(buf ^ 1);
        __syncthreads();
    }

#pragma unroll
    for (int i = 0; i < 4; ++i) {
        qs[i] += __shfl_xor(qs[i], 16, 64);
        qs[i] += __shfl_xor(qs[i], 32, 64);
    }
    const int vrr = r0 + wn * 16 + lr;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qsum = __shfl(qs[i], 4 * g + j, 64);
            const int m = m0 + wm * 64 + i * 16 + 4 * g + j;
            if (m >= c.M || vrr >= c.R) continue;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int A = shift_field(accv[0][i][f][j], f) - qsum;
                const int U = PAIR ? shift_field(accv[NB - 1][i][f][j], f) - qsum : 0;
                emit(c, m, vrr, f, A, U);
            }
        }
    }
}

// ===========================================================================
// Generic kernel: one lane per (token row, packed row), byte loads, any K.
// ===========================================================================
__global__ __launch_bounds__(256) void k_generic(Contract c) {
    const int64_t idx = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (idx >= (int64_t)c.M * c.R) return;
    const int m = (int)(idx / c.R);
    const int vr = (int)(idx % c.R);
    const int K = c.K;
    const int8_t *qr = c.q + (size_t)m * c.ldq;
    const uint8_t *pg = c.P + (size_t)vr * K;
    const uint8_t *pu = c.P + (size_t)(c.R + vr) * K;
    int A[4] = {0, 0, 0, 0}, U[4] = {0, 0, 0, 0};
    for (int k = 0; k < K; ++k) {
        const int qv = qr[k];
        const unsigned b = pg[k];
#pragma unroll
        for (int f = 0; f < 4; ++f) A[f] += qv * ((int)((b >> (2 * f)) & 3u) - 1);
        if (c.pair) {
            const unsigned bu = pu[k];
#pragma unroll
            for (int f = 0; f < 4; ++f) U[f] += qv * ((int)((bu >> (2 * f)) & 3u) - 1);
        }
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) emit(c, m, vr, f, A[f], U[f]);
}

} // namespace

hipError_t launch_gemm(const Contract &c, hipStream_t s) {
    const int ntm = (c.M + kBM - 1) / kBM;
    const int ntn = (c.R + kVR - 1) / kVR;
    if (c.pair)
        hipLaunchKernelGGL(k_gemm<true>, dim3(ntm * ntn), dim3(256), 0, s, c, ntm);
    else
        hipLaunchKernelGGL(k_gemm<false>, dim3(ntm * ntn), dim3(256), 0, s, c, ntm);
    return hipGetLastError();
}

hipError_t launch_generic(const Contract &c, hipStream_t s) {
    const int64_t n = (int64_t)c.M * c.R;
    hipLaunchKernelGGL(k_generic, dim3((unsigned)((n + 255) / 256)), dim3(256), 0, s, c);
    return hipGetLastError();
}

} // namespace bl
