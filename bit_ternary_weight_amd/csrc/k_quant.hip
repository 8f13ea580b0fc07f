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
// One workgroup (256 lanes = 4 waves) per token row.  The main kernel
// (k_rowq) reads the row once, with 16-byte loads all issued before the
// first use, and keeps it in registers for the norm, the maximum and the
// codes; every launch of it covers a whole batch of problems.  Rows that do
// not fit that shape (unaligned, or longer than 8 loads per lane) take
// k_quant_rows, which re-reads the row from L2 for each pass.  The row
// maximum is exact in any order; the fp64 sum of squares is reduced in a
// fixed tree order.
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

// Block maximum and integer sum: DPP within each wave, then one LDS-only
// barrier (no global store or load of the block need wait for it); each
// reduction uses its own LDS slots once, so no second barrier guards them.
__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max_dpp(v);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    lds_barrier();
    return fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
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

__device__ __forceinline__ int block_isum(int v, int *red) {
    v = wave_sum_dpp(v);
    int w = threadIdx.x >> 6;
    if ((threadIdx.x & 63) == 0) red[w] = v;
    lds_barrier();
    return (red[0] + red[1]) + (red[2] + red[3]);
}

// Fallback: any alignment and length; three passes over the row.
template <typename T, bool NORM, bool VEC>
__global__ __launch_bounds__(kThreads) void k_quant_rows(const T *__restrict__ x, int K, int ldx,
                                                         const float *__restrict__ g, float eps,
                                                         int8_t *__restrict__ q, float *__restrict__ a,
                                                         int *__restrict__ qsum, int tile_m) {
    __shared__ float redf[4];
    __shared__ double redd[4];
    __shared__ int redi[4];
    const int m = blockIdx.x;
    const T *row = x + (int64_t)m * ldx;
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

    int csum = 0;
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
                csum += c[i];
            }
            *reinterpret_cast<uint32_t *>(q + code_offset(m, k, K, tile_m)) = pack4(c[0], c[1], c[2], c[3]);
        }
    } else {
        for (int k = threadIdx.x; k < K; k += kThreads) {
            const int c = quant1(elem<T, NORM>(row, k, r, g), s);
            csum += c;
            q[code_offset(m, k, K, tile_m)] = (int8_t)c;
        }
    }
    if (qsum) {
        csum = block_isum(csum, redi);
        if (threadIdx.x == 0) qsum[m] = csum;
    }
}

// ---------------------------------------------------------------------------
// Register-resident quantizer.  Lane t of a row's workgroup owns the 16-byte
// chunks c * 256 + t (c < NCH) of the row: E = 16 / sizeof(T) elements each.
// All its loads (row chunks and, for RMSNorm, the matching gain chunks) are
// issued back to back, so a row costs one memory round trip; the normalized
// values stay in registers through the maximum and the code pass.  The
// arithmetic is that of k_quant_rows, element by element.
// ---------------------------------------------------------------------------
template <typename T>
__device__ __forceinline__ void unpack16(uint4 u, float *v);
template <>
__device__ __forceinline__ void unpack16<float>(uint4 u, float *v) {
    v[0] = __uint_as_float(u.x); v[1] = __uint_as_float(u.y);
    v[2] = __uint_as_float(u.z); v[3] = __uint_as_float(u.w);
}
template <>
__device__ __forceinline__ void unpack16<uint16_t>(uint4 u, float *v) {
    const uint32_t w[4] = {u.x, u.y, u.z, u.w};
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        v[2 * i] = __uint_as_float(w[i] << 16);
        v[2 * i + 1] = __uint_as_float(w[i] & 0xFFFF0000u);
    }
}

constexpr int kRowqMaxChunks = 8;

template <typename T, bool NORM, int NCH>
__global__ __launch_bounds__(kThreads) void k_rowq(QuantBatch qb) {
    constexpr int E = 16 / (int)sizeof(T);
    __shared__ float redf[4];
    __shared__ double redd[4];
    __shared__ int redi[4];
    // the problem whose [row0, row0 + M) holds this block: its index from
    // the row starts (all loaded at once), then its fields by that index
    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < qb.n && (int)blockIdx.x >= qb.p[i].row0) pi = i;
    const QuantProblem &p = qb.p[pi];
    const int m = (int)blockIdx.x - p.row0;
    const int K = p.K;
    const T *row = reinterpret_cast<const T *>(p.x) + (int64_t)m * p.ldx;
    const int t = threadIdx.x;

    uint4 raw[NCH];
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = (c * kThreads + t) * E;
        raw[c] = k < K ? *reinterpret_cast<const uint4 *>(row + k) : make_uint4(0, 0, 0, 0);
    }
    float gv[NORM ? NCH : 1][NORM ? E : 1];
    if (NORM) {
        const bool has_g = p.gain != nullptr;
#pragma unroll
        for (int c = 0; c < NCH; ++c) {
            const int k = (c * kThreads + t) * E;
#pragma unroll
            for (int h = 0; h < E / 4; ++h) {
                float4 gg = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
                if (has_g && k < K) gg = *reinterpret_cast<const float4 *>(p.gain + k + 4 * h);
                gv[c][4 * h] = gg.x; gv[c][4 * h + 1] = gg.y;
                gv[c][4 * h + 2] = gg.z; gv[c][4 * h + 3] = gg.w;
            }
        }
    }

    float v[NCH][E];
#pragma unroll
    for (int c = 0; c < NCH; ++c) unpack16<T>(raw[c], v[c]);

    if (NORM) {
        double ss = 0.0;
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int i = 0; i < E; ++i) ss += (double)v[c][i] * (double)v[c][i];
        ss = block_sum(ss, redd);
        const float r = (float)(1.0 / sqrt(ss / (double)K + (double)p.eps));
        // with no gain the factor is 1.0 and the product is exact
#pragma unroll
        for (int c = 0; c < NCH; ++c)
#pragma unroll
            for (int i = 0; i < E; ++i) v[c][i] = (v[c][i] * r) * gv[c][i];
    }

    // chunks past the row end hold zeros, which leave the maximum unchanged
    float amax = 0.0f;
#pragma unroll
    for (int c = 0; c < NCH; ++c)
#pragma unroll
        for (int i = 0; i < E; ++i) amax = fmaxf(amax, fabsf(v[c][i]));
    amax = block_max(amax, redf);
    const float s = 127.0f / fmaxf(amax, kFloor);   // IEEE fp32 division
    if (t == 0) p.a[m] = s;

    int csum = 0;
#pragma unroll
    for (int c = 0; c < NCH; ++c) {
        const int k = (c * kThreads + t) * E;
        uint32_t w[E / 4];
#pragma unroll
        for (int h = 0; h < E / 4; ++h) {
            int cc[4];
#pragma unroll
            for (int i = 0; i < 4; ++i) cc[i] = quant1(v[c][4 * h + i], s);
            csum += (cc[0] + cc[1]) + (cc[2] + cc[3]);
            w[h] = pack4(cc[0], cc[1], cc[2], cc[3]);
        }
        if (k < K) {
            int8_t *dst = p.q + code_offset(m, k, K, p.tile_m);   // 8 codes never straddle a 64-code piece
            if (E == 8) *reinterpret_cast<uint2 *>(dst) = make_uint2(w[0], w[E / 4 - 1]);
            else *reinterpret_cast<uint32_t *>(dst) = w[0];
        }
    }
    if (p.qsum) {
        // zero-filled chunks give code 0 and add nothing
        csum = block_isum(csum, redi);
        if (t == 0) p.qsum[m] = csum;
    }
}

template <typename T>
bool rowq_fits(const QuantProblem &p) {
    constexpr int E = 16 / (int)sizeof(T);
    return p.K % E == 0 && p.ldx % E == 0 && (uintptr_t)p.x % 16 == 0 && (uintptr_t)p.q % (E / 4 * 4) == 0 &&
           (p.gain == nullptr || (uintptr_t)p.gain % 16 == 0) && p.K <= kRowqMaxChunks * kThreads * E;
}

bool rowq_fits(const QuantProblem &p) {
    return p.x_dt == BL_BF16 ? rowq_fits<uint16_t>(p) : rowq_fits<float>(p);
}

template <typename T, bool NORM>
hipError_t go_rowq(QuantBatch &qb, int rows, int kmax, hipStream_t s) {
    constexpr int E = 16 / (int)sizeof(T);
    const int per = kThreads * E;
    const int nch = (kmax + per - 1) / per;
    const dim3 grid(rows), block(kThreads);
    if (nch <= 1) hipLaunchKernelGGL((k_rowq<T, NORM, 1>), grid, block, 0, s, qb);
    else if (nch <= 2) hipLaunchKernelGGL((k_rowq<T, NORM, 2>), grid, block, 0, s, qb);
    else if (nch <= 4) hipLaunchKernelGGL((k_rowq<T, NORM, 4>), grid, block, 0, s, qb);
    else hipLaunchKernelGGL((k_rowq<T, NORM, 8>), grid, block, 0, s, qb);
    return hipGetLastError();
}

// Launches one k_rowq over problems that all fit it and share dtype and norm.
hipError_t launch_rowq(QuantBatch &qb, hipStream_t s) {
    int rows = 0, kmax = 0;
    for (int i = 0; i < qb.n; ++i) {
        qb.p[i].row0 = rows;
        rows += qb.p[i].M;
        kmax = qb.p[i].K > kmax ? qb.p[i].K : kmax;
    }
    if (rows == 0) return hipSuccess;
    const bool bf = qb.p[0].x_dt == BL_BF16;
    if (qb.p[0].norm) return bf ? go_rowq<uint16_t, true>(qb, rows, kmax, s) : go_rowq<float, true>(qb, rows, kmax, s);
    return bf ? go_rowq<uint16_t, false>(qb, rows, kmax, s) : go_rowq<float, false>(qb, rows, kmax, s);
}

template <bool NORM>
hipError_t launch_rows(const void *x, int dt, int M, int K, int ldx, const float *g, float eps,
                       int8_t *q, float *a, int *qsum, hipStream_t s, int tile_m = 0) {
    // Vector path: 4 elements per access, every row start aligned for it.
    const int esz = dt == BL_BF16 ? 2 : 4;
    const bool vec = (K % 4 == 0) && (ldx % 4 == 0) && ((uintptr_t)x % (4 * esz) == 0) &&
                     ((uintptr_t)q % 4 == 0);
    dim3 grid(M), block(kThreads);
    if (dt == BL_BF16) {
        const uint16_t *xp = (const uint16_t *)x;
        if (vec)
            hipLaunchKernelGGL((k_quant_rows<uint16_t, NORM, true>), grid, block, 0, s, xp, K, ldx, g, eps, q, a, qsum, tile_m);
        else
            hipLaunchKernelGGL((k_quant_rows<uint16_t, NORM, false>), grid, block, 0, s, xp, K, ldx, g, eps, q, a, qsum, tile_m);
    } else {
        const float *xp = (const float *)x;
        if (vec)
            hipLaunchKernelGGL((k_quant_rows<float, NORM, true>), grid, block, 0, s, xp, K, ldx, g, eps, q, a, qsum, tile_m);
        else
            hipLaunchKernelGGL((k_quant_rows<float, NORM, false>), grid, block, 0, s, xp, K, ldx, g, eps, q, a, qsum, tile_m);
    }
    return hipGetLastError();
}

// One problem: k_rowq when it fits, else k_quant_rows.
hipError_t launch_one(const QuantProblem &p, hipStream_t s) {
    if (p.M <= 0) return hipSuccess;
    if (rowq_fits(p)) {
        QuantBatch qb;
        qb.n = 1;
        qb.p[0] = p;
        return launch_rowq(qb, s);
    }
    if (p.norm) return launch_rows<true>(p.x, p.x_dt, p.M, p.K, p.ldx, p.gain, p.eps, p.q, p.a, p.qsum, s, p.tile_m);
    return launch_rows<false>(p.x, p.x_dt, p.M, p.K, p.ldx, nullptr, 0.0f, p.q, p.a, p.qsum, s, p.tile_m);
}

} // namespace

hipError_t launch_quant_batch(QuantBatch &qb, hipStream_t s) {
    // one launch when every problem fits the register kernel and they share
    // dtype and norm; otherwise one launch per problem
    bool one = qb.n > 0;
    for (int i = 0; i < qb.n; ++i)
        one = one && rowq_fits(qb.p[i]) && qb.p[i].x_dt == qb.p[0].x_dt && qb.p[i].norm == qb.p[0].norm;
    if (one) return launch_rowq(qb, s);
    for (int i = 0; i < qb.n; ++i)
        if (hipError_t e = launch_one(qb.p[i], s); e != hipSuccess) return e;
    return hipSuccess;
}

hipError_t launch_quant_act(const void *x, int x_dt, int M, int K, int ldx, int8_t *q, float *a, int *qsum,
                            hipStream_t s) {
    QuantProblem p{};
    p.x = x; p.q = q; p.a = a; p.qsum = qsum; p.gain = nullptr; p.eps = 0.0f; p.norm = 0;
    p.x_dt = x_dt; p.M = M; p.K = K; p.ldx = ldx; p.row0 = 0;
    return launch_one(p, s);
}

hipError_t launch_rmsnorm_quant(const void *h, int h_dt, int M, int K, const float *g, float eps,
                                int8_t *q, float *a, int *qsum, hipStream_t s) {
    QuantProblem p{};
    p.x = h; p.q = q; p.a = a; p.qsum = qsum; p.gain = g; p.eps = eps; p.norm = 1;
    p.x_dt = h_dt; p.M = M; p.K = K; p.ldx = K; p.row0 = 0;
    return launch_one(p, s);
}

} // namespace bl
