// k_gemv.hip -- decode-path BitLinear (M <= 64 tokens): stream the packed
// ternary weights from HBM once, expand the 2-bit fields in registers, and
// contract them with the int8 activations on the matrix cores.
//
// "Transformers 实战 BitNet 1.58 位量化", section "推理侧 BitLinear：打包权重、解包与缩放":
// the inference forward quantizes the activations per token, multiplies them
// with the unpacked ternary weight and rescales by both scales; the subln
// paragraph after it places an RMSNorm before the projections that follow
// the attention and MLP activations.  Activation quantization itself is step
// 3 of section "BitLinear 的三步量化" on the same page.
//
// Work split.  A workgroup of W waves owns one tile of 16 packed rows (64
// output columns; PAIR: 16 gate rows plus the 16 matching up rows) over the
// whole K range, so no partial sums leave the workgroup.  Wave w takes the
// 64-wide k-steps w, w + W, w + 2W, ...; at any moment the W waves read W
// adjacent 64-byte pieces of the same 16 rows.  Each wave issues the loads of
// up to KSMAX steps before touching any of them, so the whole weight stream of
// the launch is in flight at once.  The W partial results are summed with LDS
// integer atomics and written by the workgroup.
//
// Prologue (modes 1, 2; M <= 4).  While the weight loads are in flight, the
// workgroup quantizes the activation rows itself (RMSNorm first in mode 2),
// reading the raw rows from L2 and keeping the codes in LDS.  Every workgroup
// derives the same codes and scales (the same fixed-order arithmetic), so a
// decode projection needs a single launch.
//
// One launch serves up to kMaxProblems independent contractions (for example
// the seven projections of a layer): blocks are numbered tile by tile across
// the problems.
#include "bl_common.h"

namespace bl {

namespace {

constexpr float kFloor = 1e-5f;

// LDS: int red[NB*MT*1024] | float a_s[64] | double rd[16] | float rf[16] | int8 q_s[M*K]
constexpr int kOffRd = 256;
constexpr int kOffRf = kOffRd + 16 * 8;
constexpr int kOffQ = kOffRf + 16 * 4 + 64;   // keeps q_s 16-byte aligned

__host__ __device__ constexpr int red_bytes(int nb, int mt) { return nb * mt * 1024 * 4; }

__device__ __forceinline__ float load1x(const void *x, int dt, size_t i) {
    return dt == BL_BF16 ? bf16_to_f32(((const uint16_t *)x)[i]) : ((const float *)x)[i];
}

// 4 consecutive elements from i (i % 4 == 0; row bases 8/16-byte aligned).
__device__ __forceinline__ void load4x(const void *x, int dt, size_t i, float v[4]) {
    if (dt == BL_BF16) {
        const uint2 t = *reinterpret_cast<const uint2 *>((const uint16_t *)x + i);
        v[0] = __uint_as_float(t.x << 16);
        v[1] = __uint_as_float(t.x & 0xFFFF0000u);
        v[2] = __uint_as_float(t.y << 16);
        v[3] = __uint_as_float(t.y & 0xFFFF0000u);
    } else {
        const float4 t = *reinterpret_cast<const float4 *>((const float *)x + i);
        v[0] = t.x; v[1] = t.y; v[2] = t.z; v[3] = t.w;
    }
}

__device__ __forceinline__ int quant1(float v, float a) {
    float r = rintf(v * a);   // fp32 product, round half to even
    r = fminf(fmaxf(r, -128.0f), 127.0f);
    return (int)r;
}

template <int W>
__device__ __forceinline__ float block_max_w(float v, float *rf) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) rf[threadIdx.x >> 6] = v;
    __syncthreads();
    float r = rf[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r = fmaxf(r, rf[i]);
    __syncthreads();
    return r;
}

template <int W>
__device__ __forceinline__ double block_sum_w(double v, double *rd) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) rd[threadIdx.x >> 6] = v;
    __syncthreads();
    double r = rd[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r += rd[i];
    __syncthreads();
    return r;
}

// Quantizes the M activation rows of problem p into q_s (LDS, [M][K]) and
// a_s.  Mode 2 applies RMSNorm first: r = float(1/sqrt(sum h^2 / K + eps))
// with the sum in fp64, then v = (h*r)*gain.  Then a = 127/max(absmax, 1e-5)
// and q = clip(round_half_even(v*a), -128, 127), all fp32.
template <int W>
__device__ void prologue(const GemvProblem &p, int tile, int8_t *q_s, float *a_s, double *rd, float *rf) {
    const int K = p.K;
    const bool vec = (K % 4 == 0) && (p.ldx % 4 == 0);
    const bool norm = p.mode == 2;
    const bool dbg = tile == 0 && p.dbg_q != nullptr;
    for (int m = 0; m < p.M; ++m) {
        const size_t row = (size_t)m * p.ldx;
        float r = 1.0f;
        if (norm) {
            double ss = 0.0;
            if (vec) {
                for (int k = threadIdx.x * 4; k < K; k += W * 256) {
                    float v[4];
                    load4x(p.x, p.x_dt, row + k, v);
#pragma unroll
                    for (int i = 0; i < 4; ++i) ss += (double)v[i] * (double)v[i];
                }
            } else {
                for (int k = threadIdx.x; k < K; k += W * 64) {
                    const double v = (double)load1x(p.x, p.x_dt, row + k);
                    ss += v * v;
                }
            }
            ss = block_sum_w<W>(ss, rd);
            r = (float)(1.0 / sqrt(ss / (double)K + (double)p.eps));
        }
        float amax = 0.0f;
        if (vec) {
            for (int k = threadIdx.x * 4; k < K; k += W * 256) {
                float v[4];
                load4x(p.x, p.x_dt, row + k, v);
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t = v[i];
                    if (norm) {
                        t = t * r;
                        if (p.gain) t = t * p.gain[k + i];
                    }
                    amax = fmaxf(amax, fabsf(t));
                }
            }
        } else {
            for (int k = threadIdx.x; k < K; k += W * 64) {
                float t = load1x(p.x, p.x_dt, row + k);
                if (norm) {
                    t = t * r;
                    if (p.gain) t = t * p.gain[k];
                }
                amax = fmaxf(amax, fabsf(t));
            }
        }
        amax = block_max_w<W>(amax, rf);
        const float s = 127.0f / fmaxf(amax, kFloor);   // IEEE fp32 division
        if (threadIdx.x == 0) {
            a_s[m] = s;
            if (dbg && p.dbg_a) p.dbg_a[m] = s;
        }
        int8_t *qrow = q_s + (size_t)m * K;
        if (vec) {
            for (int k = threadIdx.x * 4; k < K; k += W * 256) {
                float v[4];
                load4x(p.x, p.x_dt, row + k, v);
                uint32_t packed = 0;
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    float t = v[i];
                    if (norm) {
                        t = t * r;
                        if (p.gain) t = t * p.gain[k + i];
                    }
                    packed |= (uint32_t)(quant1(t, s) & 0xFF) << (8 * i);
                }
                *reinterpret_cast<uint32_t *>(qrow + k) = packed;
                if (dbg) *reinterpret_cast<uint32_t *>(p.dbg_q + (size_t)m * K + k) = packed;
            }
        } else {
            for (int k = threadIdx.x; k < K; k += W * 64) {
                float t = load1x(p.x, p.x_dt, row + k);
                if (norm) {
                    t = t * r;
                    if (p.gain) t = t * p.gain[k];
                }
                const int8_t c = (int8_t)quant1(t, s);
                qrow[k] = c;
                if (dbg) p.dbg_q[(size_t)m * K + k] = c;
            }
        }
    }
}

template <int W, int MT, int KSMAX, bool PAIR, bool FUSED>
__global__ __launch_bounds__(W * 64) void k_gemv(GemvBatch b) {
    constexpr int NB = PAIR ? 2 : 1;
    constexpr int NE = MT * 1024;
    extern __shared__ __attribute__((aligned(16))) unsigned char smem[];
    int *red = reinterpret_cast<int *>(smem);
    float *a_s = reinterpret_cast<float *>(smem + red_bytes(NB, MT));
    double *rd = reinterpret_cast<double *>(smem + red_bytes(NB, MT) + kOffRd);
    float *rf = reinterpret_cast<float *>(smem + red_bytes(NB, MT) + kOffRf);
    int8_t *q_s = reinterpret_cast<int8_t *>(smem + red_bytes(NB, MT) + kOffQ);

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < b.n && (int)blockIdx.x >= b.p[i].tile0) pi = i;
    const GemvProblem &p = b.p[pi];

    const int tile = (int)blockIdx.x - p.tile0;
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;
    const int g = lane >> 4;
    const int r0 = tile * 16;
    const int vr = r0 + lr;
    const bool row_ok = vr < p.R;
    const int K = p.K;
    const int M = p.M;
    const int nsteps = (K + 63) >> 6;
    const int ks = (nsteps + W - 1) / W;
    constexpr bool fused = FUSED;
    const int8_t *qg = reinterpret_cast<const int8_t *>(p.x);

    for (int i = threadIdx.x; i < NB * NE; i += W * 64) red[i] = 0;

    const uint8_t *pw[NB];
    pw[0] = p.P + (size_t)vr * K + 16 * g;
    if (PAIR) pw[NB - 1] = p.P + (size_t)(p.R + vr) * K + 16 * g;

    v4i accv[NB][MT][4];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int mt = 0; mt < MT; ++mt)
#pragma unroll
            for (int f = 0; f < 4; ++f) accv[t][mt][f] = v4i{0, 0, 0, 0};
    int qs[MT];
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) qs[mt] = 0;

    bool need_prologue = fused;
    for (int c0 = 0; c0 < ks; c0 += KSMAX) {
        // Issue the loads of this chunk: weights always, codes in mode 0.
        v4i bv[NB][KSMAX];
        v4i av[FUSED ? 1 : MT][KSMAX];
#pragma unroll
        for (int s = 0; s < KSMAX; ++s) {
            const int st = wave + W * (c0 + s);
            const int kk = st * 64 + 16 * g;
            const bool kok = (c0 + s) < ks && kk < K;
#pragma unroll
            for (int t = 0; t < NB; ++t)
                bv[t][s] = (kok && row_ok) ? ld16(pw[t] + st * 64) : v4i{0, 0, 0, 0};
            if (!FUSED) {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) {
                    const int m = mt * 16 + lr;
                    av[mt][s] = (kok && m < M) ? ld16(qg + (size_t)m * p.ldx + kk) : v4i{0, 0, 0, 0};
                }
            }
        }
        if (FUSED && need_prologue) {
            prologue<W>(p, tile, q_s, a_s, rd, rf);
            __syncthreads();
            need_prologue = false;
        }
#pragma unroll
        for (int s = 0; s < KSMAX; ++s) {
            v4i a_op[MT];
            if (FUSED) {
                // MT == 1: row lr of the codes kept in LDS by the prologue
                const int st = wave + W * (c0 + s);
                const int kk = st * 64 + 16 * g;
                const bool kok = (c0 + s) < ks && kk < K;
                a_op[0] = (kok && lr < M) ? *reinterpret_cast<const v4i *>(q_s + (size_t)lr * K + kk)
                                          : v4i{0, 0, 0, 0};
            } else {
#pragma unroll
                for (int mt = 0; mt < MT; ++mt) a_op[mt] = av[mt][s];
            }
#pragma unroll
            for (int mt = 0; mt < MT; ++mt) qs[mt] += rowsum16(a_op[mt]);
#pragma unroll
            for (int t = 0; t < NB; ++t) {
                v4i fb[4];
                expand(bv[t][s], fb);
#pragma unroll
                for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                    for (int f = 0; f < 4; ++f) accv[t][mt][f] = mfma16(a_op[mt], fb[f], accv[t][mt][f]);
            }
        }
    }

    // Row sums of the codes over this wave's k-steps: reduce the k-groups.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        qs[mt] += __shfl_xor(qs[mt], 16, 64);
        qs[mt] += __shfl_xor(qs[mt], 32, 64);
    }
    __syncthreads();   // red[] cleared (and the prologue's LDS settled)

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qsum = __shfl(qs[mt], 4 * g + j, 64);
            if (mt * 16 + 4 * g + j >= M) continue;
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int v = shift_field(accv[t][mt][f][j], f) - qsum;
                    atomicAdd(&red[t * NE + ((mt * 4 + f) * 4 + j) * 64 + lane], v);
                }
        }
    }
    __syncthreads();

    for (int e = threadIdx.x; e < NE; e += W * 64) {
        const int ln = e & 63;
        const int j = (e >> 6) & 3;
        const int f = (e >> 8) & 3;
        const int mt = e >> 10;
        const int m = mt * 16 + 4 * (ln >> 4) + j;
        const int vrr = r0 + (ln & 15);
        if (m >= M || vrr >= p.R) continue;
        const float a = fused ? a_s[m] : p.a[m];
        emit_out(p.y, p.y_dt, p.ldy, PAIR, p.seg, p.R, p.w_mean, m, vrr, f, a, red[e],
                 PAIR ? red[(NB - 1) * NE + e] : 0);
    }
}

template <int W, int MT, int KSMAX, bool PAIR, bool FUSED>
hipError_t go(GemvBatch &b, int tiles, size_t lds, hipStream_t s) {
    hipLaunchKernelGGL((k_gemv<W, MT, KSMAX, PAIR, FUSED>), dim3(tiles), dim3(W * 64), lds, s, b);
    return hipGetLastError();
}

template <int W, int MT, bool PAIR, bool FUSED>
hipError_t go_ks(int ksmax, GemvBatch &b, int tiles, size_t lds, hipStream_t s) {
    switch (ksmax) {
    case 1: return go<W, MT, 1, PAIR, FUSED>(b, tiles, lds, s);
    case 2: return go<W, MT, 2, PAIR, FUSED>(b, tiles, lds, s);
    case 4: return go<W, MT, 4, PAIR, FUSED>(b, tiles, lds, s);
    default: return go<W, MT, 8, PAIR, FUSED>(b, tiles, lds, s);
    }
}

// Waves per workgroup: 16 while a lane's accumulators are small, else 8
// (twice the registers per lane).
constexpr int waves_of(int mt, bool pair) { return (pair || mt >= 3) ? 8 : 16; }

template <bool PAIR, bool FUSED>
hipError_t go_mt(int mt, int ksmax, GemvBatch &b, int tiles, size_t lds, hipStream_t s) {
    if constexpr (FUSED) {
        return go_ks<waves_of(1, PAIR), 1, PAIR, FUSED>(ksmax, b, tiles, lds, s);
    } else {
        switch (mt) {
        case 1: return go_ks<waves_of(1, PAIR), 1, PAIR, FUSED>(ksmax, b, tiles, lds, s);
        case 2: return go_ks<waves_of(2, PAIR), 2, PAIR, FUSED>(ksmax, b, tiles, lds, s);
        case 3: return go_ks<waves_of(3, PAIR), 3, PAIR, FUSED>(ksmax, b, tiles, lds, s);
        default: return go_ks<waves_of(4, PAIR), 4, PAIR, FUSED>(ksmax, b, tiles, lds, s);
        }
    }
}

// Largest unroll depth (k-steps in flight per wave) that each variant holds
// in registers without spilling (from the compiler's resource report).
int max_ksmax(int mt, bool pair, bool fused) {
    if (fused) return 8;
    if (!pair) return mt == 2 ? 4 : 8;
    return mt <= 2 ? 8 : (mt == 3 ? 4 : 2);
}

} // namespace

hipError_t launch_gemv_batch(GemvBatch &b, hipStream_t s) {
    int tiles = 0, max_m = 1, max_steps = 1;
    size_t qbytes = 0;
    const bool pair = b.p[0].pair != 0;
    const bool fused = b.p[0].mode != 0;
    for (int i = 0; i < b.n; ++i) {
        GemvProblem &p = b.p[i];
        if ((p.mode != 0) != fused || (p.pair != 0) != pair) return hipErrorInvalidValue;
        p.tile0 = tiles;
        tiles += (p.R + 15) / 16;
        if (p.M > max_m) max_m = p.M;
        const int st = (p.K + 63) / 64;
        if (st > max_steps) max_steps = st;
        if (fused && (size_t)p.M * p.K > qbytes) qbytes = (size_t)p.M * p.K;
    }
    if (fused && max_m > kFuseMaxM) return hipErrorInvalidValue;
    const int mt = fused ? 1 : (max_m + 15) / 16;
    const int W = waves_of(mt, pair);
    const int ks = (max_steps + W - 1) / W;
    const int cap = max_ksmax(mt, pair, fused);
    int ksmax = 1;
    while (ksmax < ks && ksmax * 2 <= cap) ksmax *= 2;
    const size_t lds = red_bytes(pair ? 2 : 1, mt) + kOffQ + ((qbytes + 15) & ~(size_t)15);
    if (pair) return fused ? go_mt<true, true>(mt, ksmax, b, tiles, lds, s) : go_mt<true, false>(mt, ksmax, b, tiles, lds, s);
    return fused ? go_mt<false, true>(mt, ksmax, b, tiles, lds, s) : go_mt<false, false>(mt, ksmax, b, tiles, lds, s);
}

} // namespace bl
