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

#include <cstring>

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

// ===========================================================================
// Streaming variant for the fused path (M <= 4).  One 16-wave workgroup per
// CU, with two roles:
//   * 8 stream waves move the packed weights into LDS with the gfx950 direct
//     global->LDS loads (global_load_lds_dwordx4) and run the MFMAs.  Each
//     owns a ring of kRing 1 KB slots; lane l's 16 bytes land at slot + 16 l
//     and only this wave reads the slot back, so consuming a slot needs only
//     the wave's own s_waitcnt vmcnt, never a workgroup barrier.  They issue
//     their first kRing loads at once, as soon as the activation loads of
//     the quantizer waves are out.
//   * 8 quantizer waves (two per SIMD) load the activation rows and quantize
//     them into LDS.  They synchronise among themselves through LDS flags,
//     not s_barrier: a stream wave is stalled in the issue of its weight
//     loads for microseconds while the memory system is saturated, and a
//     workgroup barrier would hold the quantizer waves behind it.
// The stream waves wait for the quantizer waves' flags before their first
// MFMA.  Both roles meet at one barrier at the end, where the column sums are
// reduced, rescaled and stored.
// ===========================================================================
constexpr int kStreamWaves = 8;
constexpr int kQuantWaves = 8;
constexpr int kLdsWaves = kStreamWaves + kQuantWaves;
constexpr int kQuantLanes = kQuantWaves * 64;
constexpr int kRing = 12;            // 1 KB ring slots per stream wave
constexpr int kLdsQBytes = 12288;    // static LDS for the activation codes (M rows of pitch Kp)
constexpr int kXRegs = 8;            // 16-byte activation chunks per quantizer lane (all rows)
constexpr int kSpinMax = 1 << 22;    // bound of every flag wait (about 0.2 s)

// Count of bounded waits that expired in this file's kernels (one copy per
// device); read and cleared by wait_expired_count().
__device__ unsigned int g_wait_expired = 0;

// Input kind of a launch of the streaming kernel, shared by all its problems:
// activation dtype, RMSNorm in the prologue or not, one activation row or up
// to four.  Each kind is its own kernel: the quantizer code of the other
// kinds is never fetched.  (The streaming kernel is launched cold, its code
// evicted from L2 by the previous launch's weight stream, so every
// instruction-cache line it runs is a miss; with all kinds in one kernel the
// waves spent a fifth of their time waiting for instruction fetch.)
constexpr int kXkF32 = 1;    // fp32 activations (else bf16)
constexpr int kXkNorm = 2;   // RMSNorm before quantizing (one row)
constexpr int kXkM1 = 4;     // every problem has one activation row
__host__ __device__ constexpr bool xk_bf16(int xk) { return (xk & kXkF32) == 0; }
__host__ __device__ constexpr bool xk_norm(int xk) { return (xk & kXkNorm) != 0; }
__host__ __device__ constexpr bool xk_m1(int xk) { return (xk & (kXkM1 | kXkNorm)) != 0; }

// Activation elements per 16-byte chunk.
__host__ __device__ constexpr int x_per_chunk(int dt) { return dt == BL_BF16 ? 8 : 4; }

// Chunks per row for K elements (quantizer lane ql takes chunk c at element
// (c * lanes + ql) * per_chunk).
__host__ __device__ inline int x_chunks(int K, int dt, int lanes) {
    const int per = x_per_chunk(dt) * lanes;
    return (K + per - 1) / per;
}

// The PER activation values of a 16-byte chunk as fp32 (bf16: 8, fp32: 4).
template <int PER>
__device__ __forceinline__ void chunk_f32(const v4i &c, float *v) {
    if (PER == 8) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            v[2 * i] = __uint_as_float((uint32_t)c[i] << 16);
            v[2 * i + 1] = __uint_as_float((uint32_t)c[i] & 0xFFFF0000u);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) v[i] = __uint_as_float((uint32_t)c[i]);
    }
}

// Flags of the quantizer waves, in LDS: qflag[w] counts the steps wave w has
// published.  A wave publishes after its LDS writes (the LDS executes one
// wave's operations in order).  Waiters poll with plain loads behind a
// compiler memory clobber (a volatile or atomic LDS load would make the
// compiler wait for every weight load in flight first).
__device__ __forceinline__ void publish(int *qflag, int w, int step) {
    asm volatile("" ::: "memory");
    if ((threadIdx.x & 63) == 0) qflag[w] = step;
    asm volatile("" ::: "memory");
}

// The poll is one LDS read and scalar compares; between polls the wave
// sleeps SLEEP x 64 cycles, so that spinning waves leave the SIMD to the
// waves sharing it (the stream waves' wait is long; the quantizer waves'
// waits on each other are short).
// A wait that runs out of polls (which only a wave held off the CU for
// about 0.2 s could cause) lets the kernel finish with whatever the flags
// guard, and counts itself in g_wait_expired (a vector atomic) so that
// bl_device_errors reports the call as unreliable instead of its output
// passing silently.
template <int SLEEP>
__device__ __forceinline__ void wait_published(const int *qflag, int step) {
    static_assert(kQuantWaves == 8, "two 16-byte reads cover the flags");
    int lo = 0;
    for (int it = 0; it < kSpinMax; ++it) {
        asm volatile("" ::: "memory");
        const v4i f = *reinterpret_cast<const v4i *>(qflag);
        const v4i h = *reinterpret_cast<const v4i *>(qflag + 4);
        lo = step;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo = min(lo, min(__builtin_amdgcn_readfirstlane(f[i]), __builtin_amdgcn_readfirstlane(h[i])));
        if (lo >= step) break;
        __builtin_amdgcn_s_sleep(SLEEP);
    }
    if (lo < step && (threadIdx.x & 63) == 0) atomicAdd(&g_wait_expired, 1u);
    asm volatile("" ::: "memory");
}

// Element m of a 4-element per-row array, m uniform and run-time (selects,
// not an indexed access: that would go through scratch memory).
template <typename T>
__device__ __forceinline__ T sel4(const T *a, int m) {
    return m == 0 ? a[0] : (m == 1 ? a[1] : (m == 2 ? a[2] : a[3]));
}

// Per-row accumulator update with a uniform, run-time row index.
template <typename T, typename F>
__device__ __forceinline__ void row_update(T *acc, int m, T v, F op) {
#pragma unroll
    for (int r = 0; r < kFuseMaxM; ++r)
        if (r == m) acc[r] = op(acc[r], v);
}

// Quantizer waves: quantize the M (<= 4) rows held in xr (register j holds
// row j / E, chunk j % E of this lane) into q_s (row pitch `pitch`), with the
// same arithmetic as prologue(): optional RMSNorm (fp64 sum of squares), then
// per-row absmax, scale and codes.  With the norm, M is 1 (register j holds
// chunk j, so the gains of chunk j sit in the static registers
// gr[j*PER/4 ...], all ones when the norm has no gain).  Each wave leaves its
// share of every row's code sum in sq_s[m * kQuantWaves + qw].  Global memory
// is not touched.
template <int PER, bool NORM, bool M1>
__device__ __forceinline__ void quant_rows(const GemvProblem &p, const v4i *xr, const v4i *gr, int E, int pitch, int qw, int ql,
                           int8_t *q_s, float *a_s, int *sq_s, double *part_d, float *part_f,
                           int *qflag) {
    const int K = p.K;
    const int M = M1 ? 1 : p.M;
    // row and chunk of each register (uniform; counted up once, no divisions)
    int jrow[kXRegs], jchunk[kXRegs];
    {
        int m = 0, c = 0;
#pragma unroll
        for (int j = 0; j < kXRegs; ++j) {
            jrow[j] = m;
            jchunk[j] = c;
            if (++c == E) {
                c = 0;
                ++m;
            }
        }
    }
    auto elem0 = [&](int j) { return (jchunk[j] * kQuantLanes + ql) * PER; };
    auto row_of = [&](int j) { return jrow[j]; };
    // Registers in use: a uniform bound, so each pass leaves its unrolled
    // loop with one branch (the code of the unused registers is never
    // fetched).  Past the row end a lane's register reads as zeros, which
    // leave the maximum, the sum of squares and the code sum unchanged and
    // are not stored.
    const int nreg = M * E;
    auto reg = [&](int j) { return elem0(j) < K ? xr[j] : v4i{0, 0, 0, 0}; };
    // the norm of register j's chunk (NORM: M == 1, so chunk j, static)
    auto norm = [&](float *v, int j, float r) {
        const v4i g0 = gr[(j * (PER / 4)) % kXRegs];
        const v4i g1 = PER == 8 ? gr[(j * 2 + 1) % kXRegs] : g0;
#pragma unroll
        for (int i = 0; i < PER; ++i)
            v[i] = (v[i] * r) * __uint_as_float((uint32_t)(i < 4 ? g0[i & 3] : g1[i & 3]));
    };
    int step = 0;
    float r[kFuseMaxM] = {1.0f, 1.0f, 1.0f, 1.0f};
    // Without a gain the norm's largest |h * r| is float(max |h| * r) (the
    // rounded product is monotone in the first factor and odd): the maximum
    // travels with the sum of squares and one rendezvous is saved.
    const bool fold = NORM && p.gain == nullptr;
    float amax[kFuseMaxM] = {0.0f, 0.0f, 0.0f, 0.0f};
    if (NORM) {
        double ss[kFuseMaxM] = {0.0, 0.0, 0.0, 0.0};
        float hm = 0.0f;
#pragma unroll
        for (int j = 0; j < kXRegs; ++j) {
            if (j >= nreg) break;
            float v[PER];
            chunk_f32<PER>(reg(j), v);
            double t = 0.0;
#pragma unroll
            for (int i = 0; i < PER; ++i) {
                t += (double)v[i] * (double)v[i];
                hm = fmaxf(hm, fabsf(v[i]));
            }
            row_update(ss, row_of(j), t, [](double a, double b) { return a + b; });
        }
#pragma unroll
        for (int m = 0; m < kFuseMaxM; ++m) {
            if (m >= M) break;
            const double w = wave_sum_dpp(ss[m]);
            if ((threadIdx.x & 63) == 0) part_d[m * kQuantWaves + qw] = w;
        }
        if (fold) {
            // NORM: one row
            const float w = wave_max_dpp(hm);
            if ((threadIdx.x & 63) == 0) part_f[qw] = w;
        }
        publish(qflag, qw, ++step);
        wait_published<1>(qflag, step);
#pragma unroll
        for (int m = 0; m < kFuseMaxM; ++m) {
            if (m >= M) break;
            double t = part_d[m * kQuantWaves];
#pragma unroll
            for (int w = 1; w < kQuantWaves; ++w) t += part_d[m * kQuantWaves + w];
            r[m] = (float)(1.0 / sqrt(t / (double)K + (double)p.eps));
        }
        if (fold) {
            float t = part_f[0];
#pragma unroll
            for (int w = 1; w < kQuantWaves; ++w) t = fmaxf(t, part_f[w]);
            amax[0] = t * r[0];
        }
    }
    if (!fold) {
#pragma unroll
        for (int j = 0; j < kXRegs; ++j) {
            if (j >= nreg) break;
            float v[PER];
            chunk_f32<PER>(reg(j), v);
            const int m = row_of(j);
            if (NORM) norm(v, j, r[0]);
            float t = 0.0f;
#pragma unroll
            for (int i = 0; i < PER; ++i) t = fmaxf(t, fabsf(v[i]));
            row_update(amax, m, t, [](float a, float b) { return fmaxf(a, b); });
        }
#pragma unroll
        for (int m = 0; m < kFuseMaxM; ++m) {
            if (m >= M) break;
            const float w = wave_max_dpp(amax[m]);
            if ((threadIdx.x & 63) == 0) part_f[m * kQuantWaves + qw] = w;
        }
        publish(qflag, qw, ++step);
        wait_published<1>(qflag, step);
#pragma unroll
        for (int m = 0; m < kFuseMaxM; ++m) {
            if (m >= M) break;
            float t = part_f[m * kQuantWaves];
#pragma unroll
            for (int w = 1; w < kQuantWaves; ++w) t = fmaxf(t, part_f[m * kQuantWaves + w]);
            amax[m] = t;
        }
    }
    float s[kFuseMaxM] = {1.0f, 1.0f, 1.0f, 1.0f};
#pragma unroll
    for (int m = 0; m < kFuseMaxM; ++m) {
        if (m >= M) break;
        s[m] = 127.0f / fmaxf(amax[m], kFloor);   // IEEE fp32 division
        if (ql == 0) a_s[m] = s[m];
    }
    int qsum[kFuseMaxM] = {0, 0, 0, 0};
#pragma unroll
    for (int j = 0; j < kXRegs; ++j) {
        const int k0 = elem0(j);
        if (j >= nreg) break;
        float v[PER];
        chunk_f32<PER>(reg(j), v);
        const int m = row_of(j);
        if (NORM) norm(v, j, r[0]);
        const float scale = sel4(s, m);
        uint32_t pk[PER / 4];
        int cs = 0;
#pragma unroll
        for (int h = 0; h < PER / 4; ++h) {
            uint32_t u = 0;
            // code + 128 is an integer in [0, 255]: the byte conversion is exact
#pragma unroll
            for (int jj = 0; jj < 4; ++jj) {
                const float q = __builtin_amdgcn_fmed3f(rintf(v[4 * h + jj] * scale), -128.0f, 127.0f);
                u = __builtin_amdgcn_cvt_pk_u8_f32(q + 128.0f, jj, u);
            }
            pk[h] = u ^ 0x80808080u;   // offset binary -> two's complement bytes
            cs = __builtin_amdgcn_sdot4((int)pk[h], 0x01010101, cs, false);
        }
        row_update(qsum, m, cs, [](int a, int b) { return a + b; });
        int8_t *dst = q_s + (size_t)m * pitch + k0;
        if (k0 < K) {
            if (PER == 8) *reinterpret_cast<uint2 *>(dst) = make_uint2(pk[0], pk[PER / 4 - 1]);
            else *reinterpret_cast<uint32_t *>(dst) = pk[0];
        }
    }
#pragma unroll
    for (int m = 0; m < kFuseMaxM; ++m) {
        if (m >= M) break;
        const int t = wave_sum_dpp(qsum[m]);
        if ((threadIdx.x & 63) == 0) sq_s[m * kQuantWaves + qw] = t;
    }
    publish(qflag, qw, ++step);
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt = VM, leaving expcnt and
// lgkmcnt unconstrained: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14].
template <int VM>
struct kWaitVm {
    static_assert(VM >= 0 && VM < 64, "vmcnt is 6 bits");
    static constexpr int value = (VM & 0xF) | (0x7 << 4) | (0xF << 8) | ((VM >> 4) << 14);
};

// The weight stream is read once per launch: its loads carry the
// non-temporal hint (cache policy bit nt), so that it does not evict the
// kernel's code and the activations from L2.
__device__ __forceinline__ void dma16(const void *src, void *lds_slot) {
    __builtin_amdgcn_global_load_lds(src, lds_slot, 16, 0, 2);
}

// s_waitcnt vmcnt(n) for a wave-uniform n < 12 (the loads of one batch).
__device__ __forceinline__ void wait_vm_upto11(int n) {
    switch (__builtin_amdgcn_readfirstlane(n)) {
    case 0: __builtin_amdgcn_s_waitcnt(kWaitVm<0>::value); break;
    case 1: __builtin_amdgcn_s_waitcnt(kWaitVm<1>::value); break;
    case 2: __builtin_amdgcn_s_waitcnt(kWaitVm<2>::value); break;
    case 3: __builtin_amdgcn_s_waitcnt(kWaitVm<3>::value); break;
    case 4: __builtin_amdgcn_s_waitcnt(kWaitVm<4>::value); break;
    case 5: __builtin_amdgcn_s_waitcnt(kWaitVm<5>::value); break;
    case 6: __builtin_amdgcn_s_waitcnt(kWaitVm<6>::value); break;
    case 7: __builtin_amdgcn_s_waitcnt(kWaitVm<7>::value); break;
    case 8: __builtin_amdgcn_s_waitcnt(kWaitVm<8>::value); break;
    case 9: __builtin_amdgcn_s_waitcnt(kWaitVm<9>::value); break;
    case 10: __builtin_amdgcn_s_waitcnt(kWaitVm<10>::value); break;
    case 11: __builtin_amdgcn_s_waitcnt(kWaitVm<11>::value); break;
    default: __builtin_amdgcn_s_waitcnt(kWaitVm<0>::value); break;
    }
}

// A unit of the weight stream is 4 packed rows x kUnitK bytes (k values) of
// one tensor: 1 KB, fetched by one wave with one 16-byte-per-lane direct load.
// Lane L fetches row q = L >> 4 of the unit, 16-byte chunk (L & 15) ^ rr, where
// rr is the row's index within its wave's row group, and the bytes land at
// slot + 16 L.  Each row's 256 bytes thus arrive as two whole 128-byte lines,
// and the xor puts the 16 rows that one MFMA operand read touches on distinct
// LDS banks.
constexpr int kUnitK = 256;
constexpr int kMaxCS = 8;   // column sets (4 packed rows each) per workgroup
constexpr int kMaxTileRows = 4 * kMaxCS;

// A workgroup owns 4*CS packed rows of each of the NB tensors, over all of K.
// Its stream waves split them into row groups of RW = min(4*CS, 16) rows: a
// stream wave always works on the same row group and tensor and walks the
// k-ranges kr0, kr0 + kstep, ...  The 16 MFMA columns of a wave are its RW
// rows times 16/RW field slots: column n is row n % RW; MFMA i (of RW/4)
// takes field i*(16/RW) + n/RW of it.  One 16-byte operand read of a row thus
// feeds RW/4 MFMAs.
template <bool PAIR, int XK>
__global__ __launch_bounds__(kLdsWaves * 64)
void k_gemv_lds(GemvBatch b) {
    constexpr int NB = PAIR ? 2 : 1;
    constexpr int SW = kStreamWaves;
    constexpr bool BF = xk_bf16(XK);
    constexpr bool NORM = xk_norm(XK);
    constexpr bool M1 = xk_m1(XK);
    // Static LDS objects (distinct from the dynamic weight ring, so the
    // compiler can tell that writing them does not race the ring's loads);
    // the dynamic ring then starts after them, never at LDS address 0.
    __shared__ int red[NB * kMaxTileRows * 4 * kFuseMaxM];   // [tensor][packed row][field][row of x]
    __shared__ float a_s[kFuseMaxM];
    __shared__ int sq_s[kFuseMaxM * kQuantWaves];      // per-wave code sums of each row
    __shared__ double part_d[kFuseMaxM * kQuantWaves];
    __shared__ float part_f[kFuseMaxM * kQuantWaves];
    __shared__ __attribute__((aligned(16))) int qflag[kQuantWaves];
    __shared__ __attribute__((aligned(16))) int xgo[kQuantWaves];   // quantizer wave w has issued its loads
    __shared__ __attribute__((aligned(16))) int8_t q_s[kLdsQBytes];
    __shared__ float wm_s[BL_MAX_SEGMENTS];
    extern __shared__ __attribute__((aligned(16))) unsigned char ring_lds[];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < b.n && (int)blockIdx.x >= b.p[i].tile0) pi = i;
    const GemvProblem &p = b.p[pi];

    const int CS = p.cs;                 // 1, 2, 4 or 8; CS * NB divides SW
    const int tile = (int)blockIdx.x - p.tile0;
    const int r0 = tile * 4 * CS;        // first packed row of the tile
    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int K = p.K;
    const int M = M1 ? 1 : p.M;
    const int Kp = (K + kUnitK - 1) / kUnitK * kUnitK;   // row pitch of q_s

    // LDS that is accumulated into or polled, and the zero tail of every code
    // row (k in [K, Kp) multiplies weight bytes that lie past K or are not
    // loaded at all), before any wave can touch it
    for (int i = threadIdx.x; i < NB * kMaxTileRows * 4 * kFuseMaxM; i += kLdsWaves * 64) red[i] = 0;
    if ((int)threadIdx.x < kQuantWaves) {
        qflag[threadIdx.x] = 0;
        xgo[threadIdx.x] = 0;
    }
    if (Kp > K)
        for (int i = threadIdx.x; i < M * (Kp - K); i += kLdsWaves * 64)
            q_s[(i / (Kp - K)) * Kp + K + i % (Kp - K)] = 0;
    lds_barrier();

    if (wave >= SW) {
        // ---------------- quantizer waves ----------------
        const int qw = wave - SW;
        const int ql = (int)threadIdx.x - SW * 64;
        constexpr int per = BF ? 8 : 4;
        constexpr int esz = BF ? 2 : 4;
        const int E = x_chunks(K, BF ? BL_BF16 : BL_F32, kQuantLanes);
        // Registers past the rows are loaded too (straight-line code), each
        // lane from its own chunk of row 0: every workgroup runs this at the
        // same moment, and placeholder loads of one fixed address would all
        // queue on the single L2 channel that holds it.
        v4i xr[kXRegs];
        v4i gr[kXRegs];
        // (lane offsets below the largest power of two in the row's bytes:
        // a mask, no division; K % 16 == 0, so the row has at least 32 bytes)
        const int rowb = K * esz;
        const size_t spread = (size_t)((ql * 16) & ((1 << (31 - __builtin_clz(rowb))) - 1));
        {
            int m = 0, c = 0;   // row and chunk of register j (no divisions)
#pragma unroll
            for (int j = 0; j < kXRegs; ++j) {
                const int k0 = (c * kQuantLanes + ql) * per;
                const bool ok = j < M * E && k0 < K;
                xr[j] = ld16((const unsigned char *)p.x + (ok ? ((size_t)m * p.ldx + k0) * esz : spread));
                if (++c == E) {
                    c = 0;
                    ++m;
                }
            }
        }
        // RMSNorm gains of this lane's chunks (shared by the rows): register
        // c*per/4 + h holds gain[k0(c) + 4h .. +3]; all ones without gains
        const bool gains = NORM && p.gain != nullptr;
        if (gains) {
            const int gspread = (ql * 4) & ((1 << (31 - __builtin_clz(K))) - 1);
#pragma unroll
            for (int j = 0; j < kXRegs; ++j) {
                const int c = j / (per / 4);
                const int h = j - c * (per / 4);
                const int k0 = (c * kQuantLanes + ql) * per + 4 * h;
                gr[j] = ld16(p.gain + (c < E && k0 < K ? k0 : gspread));
            }
        } else {
#pragma unroll
            for (int j = 0; j < kXRegs; ++j) gr[j] = v4i{0x3F800000, 0x3F800000, 0x3F800000, 0x3F800000};
        }
        const int nscale = PAIR ? 2 : p.seg.n;
        const float wmv = ql < nscale ? p.w_mean[ql] : 0.0f;
        // The activation loads are now in the memory queues: the stream waves
        // may start (issued behind the weight stream instead, they would
        // return only after most of it).
        asm volatile("" ::: "memory");
        if ((threadIdx.x & 63) == 0) xgo[qw] = 1;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>::value);
        if (ql < nscale) wm_s[ql] = wmv;
        quant_rows<per, NORM, M1>(p, xr, gr, E, Kp, qw, ql, q_s, a_s, sq_s, part_d, part_f, qflag);
    } else {
        // ---------------- stream waves ----------------
        const int lr = lane & 15;
        const int g = lane >> 4;
        const int nkr = Kp / kUnitK;
        // every count here is a power of two: shifts and masks, no divisions
        const int lcs = CS >= 8 ? 3 : (CS >= 4 ? 2 : (CS >= 2 ? 1 : 0));   // log2 CS
        const int lrw = lcs + 2 < 4 ? lcs + 2 : 4;   // log2 of the rows per row group
        const int RW = 1 << lrw;
        const int lupk = lrw - 2;                    // log2 of the units per k-range
        const int UPK = 1 << lupk;
        const int lgrp = (lcs + 2 - lrw) + (NB == 2 ? 1 : 0);   // log2 of the stream waves per k-range
        const int tsel = wave & (NB - 1);            // tensor of this wave
        const int rg = (wave >> (NB == 2 ? 1 : 0)) & ((1 << (lcs + 2 - lrw)) - 1);   // row group of this wave
        const int kr0 = wave >> lgrp;
        const int kstep = SW >> lgrp;
        const int ks = kr0 < nkr ? ((nkr - kr0 + kstep - 1) >> (3 - lgrp)) : 0;   // k-ranges of this wave
        const int kb = kRing >> lupk;                // k-ranges per batch (kRing is a multiple of 4)
        unsigned char *ring = ring_lds + (size_t)wave * (kRing * 1024);
        const int row0 = r0 + rg * RW;               // first packed row of the row group

        // this lane's share of a unit load: row q of the unit, swizzled chunk
        const int dq = lane >> 4;
        const int dpc = lane & 15;
        // this lane's MFMA column: row rr of the group, field slot fs
        const int rr = lr & (RW - 1);
        const int fs = lr >> lrw;
        const int8_t *qrow = q_s + (size_t)(lr < M ? lr : 0) * Kp + 16 * g;
        v4i acc[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = v4i{0, 0, 0, 0};

        // Batches of kb k-ranges: issue every unit of the batch, then consume
        // the k-ranges in order, each once its own units have landed.  (A
        // wait per k-range of UPK units; waiting unit by unit slowed the whole
        // stream down on this hardware.)  The first weight load goes out
        // only after every quantizer wave has issued its activation loads.
        wait_published<1>(xgo, 1);
        for (int b0 = 0; b0 < ks; b0 += kb) {
            const int nb = ks - b0 < kb ? ks - b0 : kb;
            for (int t = 0; t < nb * UPK; ++t) {
                const int kr = kr0 + kstep * (b0 + (t >> lupk));
                const int u = t & (UPK - 1);
                const int row = row0 + 4 * u + dq;
                const int lc = dpc ^ ((4 * u + dq) & 15);
                const bool ok = row < p.R && kr * kUnitK + 16 * lc < K;
                const uint8_t *src = ok ? p.P + (size_t)(tsel * p.R + row) * K + (size_t)kr * kUnitK + 16 * lc
                                        : p.P + 16 * dpc;
                dma16(src, ring + t * 1024);
            }
            for (int t = 0; t < nb; ++t) {
                // this k-range's units have landed (loads complete in order)
                wait_vm_upto11((nb - 1 - t) << lupk);
                // the activation codes (once; the quantizer waves publish once per
                // reduction -- the norm's sum of squares, the absmax unless it
                // travels with the sum -- and once when done)
                if (b0 == 0 && t == 0) wait_published<4>(qflag, NORM && p.gain != nullptr ? 3 : 2);
                const int kr = kr0 + kstep * (b0 + t);
                const unsigned char *slot = ring + (t * UPK + (rr >> 2)) * 1024 + 256 * (rr & 3);
                // all operand reads of the k-range first: one LDS round trip
                v4i bw[4], av[4];
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    bw[j] = *reinterpret_cast<const v4i *>(slot + 16 * ((4 * j + g) ^ rr));
                    av[j] = lr < M ? *reinterpret_cast<const v4i *>(qrow + kr * kUnitK + 64 * j) : v4i{0, 0, 0, 0};
                }
                if (RW == 16) {
                    // all four fields of every byte: masked in place they
                    // are the codes + 1 times 1, 4, 16 and (after >> 2) 16,
                    // a scale the reduction divides out exactly
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        v4i f0, f1, f2, f3;
#pragma unroll
                        for (int d = 0; d < 4; ++d) {
                            const uint32_t w = (uint32_t)bw[j][d];
                            f0[d] = (int)(w & 0x03030303u);
                            f1[d] = (int)(w & 0x0C0C0C0Cu);
                            f2[d] = (int)(w & 0x30303030u);
                            f3[d] = (int)((w >> 2) & 0x30303030u);
                        }
                        acc[0] = mfma16(av[j], f0, acc[0]);
                        acc[1] = mfma16(av[j], f1, acc[1]);
                        acc[2] = mfma16(av[j], f2, acc[2]);
                        acc[3] = mfma16(av[j], f3, acc[3]);
                    }
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
#pragma unroll
                        for (int i = 0; i < 2; ++i) {
                            if (i >= UPK) break;
                            const int fsh = 2 * (i * (16 / RW) + fs);
                            v4i fb;
#pragma unroll
                            for (int d = 0; d < 4; ++d) fb[d] = (int)(((uint32_t)bw[j][d] >> fsh) & 0x03030303u);
                            acc[i] = mfma16(av[j], fb, acc[i]);
                        }
                    }
                }
            }
        }

        // 4. column sums across the waves of a row group.  Lanes 0-15 hold
        // rows 0-3 of each 16 x 16 result (row j in element j), column = lane.
        if (lane < 16) {
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                if (i >= UPK) break;
                const int prow = rg * RW + rr;          // packed row within the tile
                const int f = i * (16 / RW) + fs;       // field
                // undo the field scale of the masked path (exact: every
                // product carries the factor)
                const int sh = RW == 16 ? (i == 0 ? 0 : (i == 1 ? 2 : 4)) : 0;
#pragma unroll
                for (int j = 0; j < kFuseMaxM; ++j)
                    if (j < M) atomicAdd(&red[((tsel * kMaxTileRows + prow) * 4 + f) * kFuseMaxM + j], acc[i][j] >> sh);
            }
        }
    }
    lds_barrier();

    // 5. rescale and store (both roles): e = (packed row, field, row of x)
    for (int e = threadIdx.x; e < 4 * CS * 4 * kFuseMaxM; e += kLdsWaves * 64) {
        const int m = e & (kFuseMaxM - 1);
        const int f = (e >> 2) & 3;
        const int prow = e >> 4;
        const int vr = r0 + prow;
        if (m >= M || vr >= p.R) continue;
        // the codes were taken as c + 1: subtract the row's code sum once
        int qsum = 0;
#pragma unroll
        for (int w = 0; w < kQuantWaves; ++w) qsum += sq_s[m * kQuantWaves + w];
        const int A = red[((0 * kMaxTileRows + prow) * 4 + f) * kFuseMaxM + m] - qsum;
        const int U = PAIR ? red[((1 * kMaxTileRows + prow) * 4 + f) * kFuseMaxM + m] - qsum : 0;
        emit_out(p.y, p.y_dt, p.ldy, PAIR, p.seg, p.R, wm_s, m, vr, f, a_s[m], A, U);
    }
    // The first tile's workgroup hands out its activation codes and scales
    // (stage outputs for checks).
    if (tile == 0 && p.dbg_q != nullptr) {
        for (int i = threadIdx.x; i < M * K; i += kLdsWaves * 64) p.dbg_q[i] = q_s[(i / K) * Kp + i % K];
        if (p.dbg_a != nullptr && (int)threadIdx.x < M) p.dbg_a[threadIdx.x] = a_s[threadIdx.x];
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

// Streaming variant (fused path, every problem's rows in kXChunks register
// chunks): problems ordered by decreasing K so the longest tiles start first.
// Even share of the batch's weight bytes per workgroup at one workgroup per
// CU.  The launcher gives each problem the largest number of column sets (4
// packed rows each) of 8, 4, 2, 1 whose tile (NB tensors x 4*CS rows x K
// bytes) stays within 1.25x this share, so every workgroup of the launch is
// resident at once and none streams much longer than the others.
size_t even_share(const GemvBatch &b, int nb, int cus) {
    size_t total = 0;
    for (int i = 0; i < b.n; ++i) total += (size_t)nb * b.p[i].R * b.p[i].K;
    return total / (size_t)cus;
}

template <bool PAIR, int XK>
hipError_t launch_lds(GemvBatch &b, hipStream_t s) {
    constexpr int NB = PAIR ? 2 : 1;
    const int cus = device_cu_count();
    const size_t share = even_share(b, NB, cus) * 5 / 4;
    GemvBatch o = b;
    int order[kMaxProblems];
    for (int i = 0; i < b.n; ++i) order[i] = i;
    for (int i = 1; i < b.n; ++i)
        for (int j = i; j > 0 && b.p[order[j]].K > b.p[order[j - 1]].K; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    int tiles = 0;
    for (int i = 0; i < b.n; ++i) {
        GemvProblem &q = o.p[i];
        q = b.p[order[i]];
        int cs = kStreamWaves / NB;   // CS * NB must divide the stream waves
        while (cs > 1 && (size_t)NB * 4 * cs * q.K > share) cs >>= 1;
        q.cs = cs;
        q.tile0 = tiles;
        tiles += (q.R + 4 * cs - 1) / (4 * cs);
    }
    o.ring_off = 0;
    const size_t lds = (size_t)kStreamWaves * kRing * 1024;   // dynamic part: the weight ring
    // Dynamic LDS above the default 64 KiB must be allowed per kernel (the
    // static part, about 17 KiB, comes on top; both fit the 160 KiB).
    if (hipError_t e = allow_dynamic_lds((const void *)k_gemv_lds<PAIR, XK>, lds); e != hipSuccess) return e;
    hipLaunchKernelGGL((k_gemv_lds<PAIR, XK>), dim3(tiles), dim3(kLdsWaves * 64), lds, s, o);
    return hipGetLastError();
}

// Input kind of a problem of the fused path.
int xkind_of(const GemvProblem &p) {
    return (p.x_dt == BL_BF16 ? 0 : kXkF32) | (p.mode == 2 ? kXkNorm : 0) | (p.M == 1 ? kXkM1 : 0);
}

// ===========================================================================
// One-row streaming kernel (M == 1): the fused decode path for a single
// activation row.  One 16-wave workgroup per CU, with the two roles of
// k_gemv_lds:
//   * 8 quantizer waves (waves 0-7: a workgroup's waves are launched in
//     order, so their row loads leave the CU before any weight load; as
//     waves 8-15 the step took 6.47 instead of 6.21 us) load the row and
//     quantize it into LDS (quant_rows: RMSNorm sum of squares, absmax,
//     codes, synchronised among themselves through LDS flags).  They issue
//     no weight load, so nothing holds them up: a wave that issues weight
//     loads is stalled in the issue for microseconds while the CU's requests
//     drain at its share of HBM.
//   * 8 stream waves (8-15) issue their weight units once the activation
//     loads are out: a unit is 4 packed rows x 256 bytes of one tensor (two whole
//     128-byte lines per row), 16 bytes per lane, loaded into registers with
//     the non-temporal hint.  Once the codes are published they consume the
//     units in order, each as soon as it has landed.  Lane (g, l) = (L >> 4,
//     L & 15) holds row l >> 2 of the unit, 16-byte chunk (l & 3) + 4 g of the
//     k-range, and reads the activation codes of the same chunk.  The four
//     2-bit fields, masked in place (codes + 1 times 1, 4, 16, 16), each go
//     through one v_mfma_i32_16x16x64_i8 with the weights as the first operand
//     (MFMA row l = unit row l >> 2, k-slice l & 3) and the codes as the
//     second (column j holds k-slice j): entry (4 r + s, s) of the product is
//     row r's sum over k-slice s, and the four slices of a row sit in the
//     four lanes of one quad, summed with DPP at the end.  Per weight dword
//     that is 5 VALU operations (the masks) instead of 9 with dot4 products;
//     the matrix core's unused 15/16 cost nothing, it is otherwise idle.
// Both roles meet at one barrier, after which the outputs are rescaled and
// stored.
// ===========================================================================
constexpr int kV1MaxUnits = 16;   // weight units per stream wave, all in flight (4 VGPRs each)
constexpr int kV1MaxRows = 32;    // packed rows per tensor per workgroup (4 * CS, NB * CS <= 8)

__device__ __forceinline__ v4i ld16_nt(const uint8_t *p) {
    return __builtin_nontemporal_load(reinterpret_cast<const v4i *>(p));
}

// Entry m (0 .. 3, per lane) of a 4-vector, with selects.
__device__ __forceinline__ int sel4_v(const v4i &a, int m) {
    return m == 0 ? a[0] : (m == 1 ? a[1] : (m == 2 ? a[2] : a[3]));
}

template <bool PAIR, int XK, int NS>
__global__ __launch_bounds__(kLdsWaves * 64)
void k_gemv_v1(GemvBatch b) {
    constexpr int NB = PAIR ? 2 : 1;
    constexpr int SW = kStreamWaves;
    constexpr bool BF = xk_bf16(XK);
    constexpr bool NORM = xk_norm(XK);
    static_assert(xk_m1(XK), "one activation row");
    __shared__ int red[NB * kV1MaxRows * 4];          // [tensor][packed row][field]
    __shared__ float a_s[kFuseMaxM];
    __shared__ int sq_s[kFuseMaxM * kQuantWaves];     // per-wave code sums
    __shared__ double part_d[kFuseMaxM * kQuantWaves];
    __shared__ float part_f[kFuseMaxM * kQuantWaves];
    __shared__ __attribute__((aligned(16))) int qflag[kQuantWaves];
    __shared__ __attribute__((aligned(16))) int xgo[kQuantWaves];   // quantizer wave w has issued its loads
    __shared__ float wm_s[BL_MAX_SEGMENTS];
    __shared__ __attribute__((aligned(16))) int8_t q_s[kLdsQBytes];

    int pi = 0;
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i)
        if (i < b.n && (int)blockIdx.x >= b.p[i].tile0) pi = i;
    const GemvProblem &p = b.p[pi];

    const int tid = threadIdx.x;
    // waves 0 .. kQuantWaves - 1 quantize, the rest stream: the quantizer
    // waves are launched first, so the activation loads leave the CU first
    const int wave = __builtin_amdgcn_readfirstlane(tid >> 6);   // uniform: scalar branches
    const int sid = tid - kQuantWaves * 64;                      // stream-wave thread index
    const int lane = tid & 63;
    const int K = p.K;
    const int R = p.R;
    const int CS = p.cs;                 // 1 .. 8, NB * CS <= 8
    const int r0 = ((int)blockIdx.x - p.tile0) * 4 * CS;
    const int nkr = (K + kUnitK - 1) / kUnitK;
    const int Kp = nkr * kUnitK;         // row pitch of q_s
    // The fields both roles need before their first global load, read here
    // together: left to itself the compiler issues each kernel-argument load
    // next to its first use, which put three dependent round trips ahead of
    // the first weight load.  (Later reads of these fields reuse the values.)
    {
        const uint8_t *P = p.P;
        const void *X = p.x;
        const float *WM = p.w_mean;
        const int nseg = p.seg.n;
        asm volatile("" ::"s"(K), "s"(R), "s"(CS), "s"(r0), "s"(P), "s"(X), "s"(WM), "s"(nseg));
    }

    // LDS that is accumulated into or polled, and the zero code tail (k in
    // [K, Kp): weight bytes there are placeholders or past K and must meet
    // code 0), before any wave can touch it
    for (int i = tid; i < NB * kV1MaxRows * 4; i += kLdsWaves * 64) red[i] = 0;
    if (tid < kQuantWaves) {
        qflag[tid] = 0;
        xgo[tid] = 0;
    }
    if (tid < Kp - K) q_s[K + tid] = 0;
    lds_barrier();

    // The epilogue's per-output constants (column, w_mean / a, the row's
    // code sum), formed by the storing threads while their weight units are
    // still arriving rather than after the final barrier.
    int ep_col = 0, ep_qsum = 0;
    float ep_s0 = 0.0f, ep_s1 = 0.0f;

    if (wave < kQuantWaves) {
        // ---------------- quantizer waves ----------------
        constexpr int per = BF ? 8 : 4;
        constexpr int esz = BF ? 2 : 4;
        const int qw = wave;
        const int ql = tid;
        const int E = x_chunks(K, BF ? BL_BF16 : BL_F32, kQuantLanes);
        v4i xr[kXRegs];
        v4i gr[kXRegs];
        // registers past the row read an in-row chunk of this lane (below
        // the largest power of two in the row's bytes; a mask, no division)
        const size_t spread = (size_t)((ql * 16) & ((1 << (31 - __builtin_clz(K * esz))) - 1));
#pragma unroll
        for (int j = 0; j < kXRegs; ++j) {
            const int k0 = (j * kQuantLanes + ql) * per;
            xr[j] = ld16((const unsigned char *)p.x + (j < E && k0 < K ? (size_t)k0 * esz : spread));
        }
        if (NORM && p.gain != nullptr) {
            const int gspread = (ql * 4) & ((1 << (31 - __builtin_clz(K))) - 1);
#pragma unroll
            for (int j = 0; j < kXRegs; ++j) {
                const int c = j / (per / 4);
                const int h = j - c * (per / 4);
                const int k0 = (c * kQuantLanes + ql) * per + 4 * h;
                gr[j] = ld16(p.gain + (c < E && k0 < K ? k0 : gspread));
            }
        } else {
#pragma unroll
            for (int j = 0; j < kXRegs; ++j) gr[j] = v4i{0x3F800000, 0x3F800000, 0x3F800000, 0x3F800000};
        }
        const int nscale = PAIR ? 2 : p.seg.n;
        const float wmv = ql < nscale ? p.w_mean[ql] : 0.0f;
        // the activation loads are in the queue: the stream waves may start
        asm volatile("" ::: "memory");
        if (lane == 0) xgo[qw] = 1;
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_waitcnt(kWaitVm<0>::value);
        if (ql < nscale) wm_s[ql] = wmv;
        quant_rows<per, NORM, true>(p, xr, gr, E, Kp, qw, ql, q_s, a_s, sq_s, part_d, part_f, qflag);
    } else {
        // ---------------- stream waves ----------------
        // tensor tsel, row group rg (4 packed rows), k-ranges kr0, kr0 +
        // kstep, ... (all counts powers of two)
        const int wave = __builtin_amdgcn_readfirstlane(sid >> 6);   // stream wave 0 .. SW - 1
        const int groups = NB * CS;
        const int lwpg = __builtin_ctz(SW / groups);   // log2 stream waves per row group
        const int grp = wave >> lwpg;
        const int tsel = NB == 2 ? (grp & 1) : 0;
        const int rg = NB == 2 ? (grp >> 1) : grp;
        const int kr0 = wave & ((1 << lwpg) - 1);
        const int kstep = 1 << lwpg;
        const int ks = kr0 < nkr ? (nkr - kr0 + kstep - 1) >> lwpg : 0;   // <= NS
        // Unit t covers the wave's k-range (t + rot) mod ks: waves and
        // workgroups start at different k-ranges, so the requests in flight at
        // any moment do not all fall on the same offsets of their rows (and on
        // the same memory channels).  The sum does not depend on the order.
        const int rot = ks > 0 ? (int)(((unsigned)blockIdx.x * 7u + (unsigned)wave * 3u) % (unsigned)ks) : 0;
        auto kr_of = [&](int t) {
            const int j = t + rot;
            return kr0 + kstep * (j >= ks ? j - ks : j);
        };
        const int lr = (lane & 15) >> 2;           // row of the unit
        const int lc = (lane & 3) + 4 * (lane >> 4);   // 16-byte chunk of the k-range
        const int row = r0 + rg * 4 + lr;
        const size_t tbytes = (size_t)R * K;       // one tensor
        // placeholder offset inside the tensor (largest power of two <= its size)
        const int lpw = 63 - __builtin_clzll((unsigned long long)tbytes);
        const size_t spread = (size_t)(16 * lane) & ((((size_t)1) << lpw) - 1);
        const uint8_t *wrow = p.P + ((size_t)tsel * R + (row < R ? row : 0)) * K;
        const uint8_t *wbase = p.P + (size_t)tsel * tbytes;
        auto unit_src = [&](int kr) {
            const int kb = kr * kUnitK + 16 * lc;
            return row < R && kb < K ? wrow + kb : wbase + spread;
        };
        // Every stream wave issues exactly NS unit loads (NS >= ks for every
        // wave of the launch): the load count is then the same on every path,
        // so the compiler's own waits for these registers are exact (a count
        // that varied by path would make it wait for all loads before the
        // first use).  Loads past ks re-read the lane's last unit (a cache hit).
        // The first unit goes out at once; the rest only after every
        // quantizer wave has issued its activation loads (one unit ahead of
        // them measured 0.1 us faster per step, two units slower).
        v4i wv[NS];
        auto load_unit = [&](int t) {
            const int tt = t < ks ? t : ks - 1;
            wv[t] = ld16_nt(tt >= 0 ? unit_src(kr_of(tt)) : wbase + spread);
        };
        load_unit(0);
        wait_published<1>(xgo, 1);
#pragma clang loop unroll(full)
        for (int t = 1; t < NS; ++t) load_unit(t);
        // the activation codes (the quantizer waves publish once per
        // reduction -- the norm's sum of squares, the absmax unless it travels
        // with the sum -- and once when done)
        wait_published<4>(qflag, NORM && p.gain != nullptr ? 3 : 2);
        if (sid < 4 * CS * 4) {
            const int f = sid & 3;
            const int vr = r0 + (sid >> 2);
#pragma unroll
            for (int w = 0; w < kQuantWaves; ++w) ep_qsum += sq_s[w];
            const float av = a_s[0];
            if (PAIR) {
                ep_col = f * R + vr;
                ep_s0 = wm_s[0] / av;   // IEEE fp32 division, as the oracle
                ep_s1 = wm_s[1] / av;
            } else {
                const ColOf co = col_of(p.seg, vr < R ? vr : 0, f);
                ep_col = co.col;
                ep_s0 = wm_s[co.seg] / av;
            }
        }
        v4i acc[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) acc[f] = v4i{0, 0, 0, 0};
        // unit t is used once the t + 1 oldest unit loads have landed (the
        // compiler's wait: vmcnt(NS - 1 - t), loads complete in order)
#pragma clang loop unroll(full)
        for (int t = 0; t < NS; ++t) {
            if (t < ks) {
                const v4i w = wv[t];
                const v4i xq = *reinterpret_cast<const v4i *>(q_s + kr_of(t) * kUnitK + 16 * lc);
                v4i f0, f1, f2, f3;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t u = (uint32_t)w[d];
                    f0[d] = (int)(u & 0x03030303u);
                    f1[d] = (int)(u & 0x0C0C0C0Cu);
                    f2[d] = (int)(u & 0x30303030u);
                    f3[d] = (int)((u >> 2) & 0x30303030u);
                }
                acc[0] = mfma16(f0, xq, acc[0]);
                acc[1] = mfma16(f1, xq, acc[1]);
                acc[2] = mfma16(f2, xq, acc[2]);
                acc[3] = mfma16(f3, xq, acc[3]);
            }
        }
        // Lane 16 r + s holds row r's k-slice s in entry s of each field's
        // product (s < 4): pick it, sum the quad (DPP), and divide the field
        // scale out exactly (every product carries it).
        const int s4 = lane & 3;
        const int acc0 = quad_sum(sel4_v(acc[0], s4));
        const int acc1 = quad_sum(sel4_v(acc[1], s4)) >> 2;
        const int acc2 = quad_sum(sel4_v(acc[2], s4)) >> 4;
        const int acc3 = quad_sum(sel4_v(acc[3], s4)) >> 4;
        if ((lane & 15) == 0 && ks > 0) {
            int *dst = red + (tsel * kV1MaxRows + rg * 4 + (lane >> 4)) * 4;
            atomicAdd(dst + 0, acc0);
            atomicAdd(dst + 1, acc1);
            atomicAdd(dst + 2, acc2);
            atomicAdd(dst + 3, acc3);
        }
    }
    lds_barrier();

    // rescale and store: thread e < 4 CS * 4 (all in stream waves 0 and 1)
    // owns output e = (packed row, field); the codes were taken as c + 1, so
    // the row's code sum comes off once
    const float a = a_s[0];
    if (sid >= 0 && sid < 4 * CS * 4 && r0 + (sid >> 2) < R) {
        const int f = sid & 3;
        const int prow = sid >> 2;
        const int A = red[(0 * kV1MaxRows + prow) * 4 + f] - ep_qsum;
        if (PAIR) {
            const int U = red[(1 * kV1MaxRows + prow) * 4 + f] - ep_qsum;
            const float pv = relu2_mul((float)A * ep_s0, (float)U * ep_s1);
            if (p.y_dt == BL_BF16) ((uint16_t *)p.y)[ep_col] = f32_to_bf16(pv);
            else ((float *)p.y)[ep_col] = pv;
        } else {
            store_out(p.y, p.y_dt, ep_col, A, ep_s0);
        }
    }
    // The first tile's workgroup hands out the codes and scale (stage outputs
    // for checks).
    if ((int)blockIdx.x == p.tile0 && p.dbg_q != nullptr) {
        for (int i = tid; i < K; i += kLdsWaves * 64) p.dbg_q[i] = q_s[i];
        if (p.dbg_a != nullptr && tid == 0) p.dbg_a[0] = a;
    }
}

template <bool PAIR, int XK, int NS>
hipError_t go_v1(GemvBatch &o, int tiles, hipStream_t s) {
    hipLaunchKernelGGL((k_gemv_v1<PAIR, XK, NS>), dim3(tiles), dim3(kLdsWaves * 64), 0, s, o);
    return hipGetLastError();
}

template <bool PAIR, int XK>
hipError_t launch_v1(GemvBatch &b, hipStream_t s) {
    constexpr int NB = PAIR ? 2 : 1;
    const int cus = device_cu_count();
    // Even share of the weight bytes per CU; each problem's tile is the
    // largest 4 * CS rows (CS = 8 / NB, ..., 1) that stays within 1.25x the
    // share; CS shrinks further until no stream wave has more than
    // kV1MaxUnits units (a row group's k-ranges split over 8 / (NB * CS)
    // waves).  Problems with the largest tiles take the lowest workgroup
    // numbers: the device dispatches those first, and the last-dispatched
    // workgroups, which can start microseconds late, get the smallest tiles.
    const size_t share = even_share(b, NB, cus) * 5 / 4;
    GemvBatch o = b;
    int csv[kMaxProblems];
    size_t tb[kMaxProblems];
    int ns = 1;
    for (int i = 0; i < b.n; ++i) {
        const GemvProblem &q = b.p[i];
        const int nkr = (q.K + kUnitK - 1) / kUnitK;
        auto units = [&](int cs) {
            const int kstep = kStreamWaves / (NB * cs);
            return (nkr + kstep - 1) / kstep;
        };
        int cs = kStreamWaves / NB;
        while (cs > 1 && ((size_t)NB * 4 * cs * q.K > share || units(cs) > kV1MaxUnits)) cs >>= 1;
        if (units(cs) > kV1MaxUnits) return hipErrorInvalidValue;   // K beyond the one-row kernel
        csv[i] = cs;
        tb[i] = (size_t)NB * 4 * cs * q.K;
        ns = units(cs) > ns ? units(cs) : ns;
    }
    int order[kMaxProblems];
    for (int i = 0; i < b.n; ++i) order[i] = i;
    for (int i = 1; i < b.n; ++i)
        for (int j = i; j > 0 && tb[order[j]] > tb[order[j - 1]]; --j) {
            const int t = order[j];
            order[j] = order[j - 1];
            order[j - 1] = t;
        }
    int tiles = 0;
    for (int i = 0; i < b.n; ++i) {
        GemvProblem &q = o.p[i];
        q = b.p[order[i]];
        q.cs = csv[order[i]];
        q.tile0 = tiles;
        tiles += (q.R + 4 * q.cs - 1) / (4 * q.cs);
    }
    o.ring_off = 0;
    switch (ns) {
    case 1: return go_v1<PAIR, XK, 1>(o, tiles, s);
    case 2: return go_v1<PAIR, XK, 2>(o, tiles, s);
    case 3: return go_v1<PAIR, XK, 3>(o, tiles, s);
    case 4: return go_v1<PAIR, XK, 4>(o, tiles, s);
    case 5: return go_v1<PAIR, XK, 5>(o, tiles, s);
    case 6: return go_v1<PAIR, XK, 6>(o, tiles, s);
    case 7: return go_v1<PAIR, XK, 7>(o, tiles, s);
    case 8: return go_v1<PAIR, XK, 8>(o, tiles, s);
    case 9: case 10: return go_v1<PAIR, XK, 10>(o, tiles, s);
    case 11: case 12: return go_v1<PAIR, XK, 12>(o, tiles, s);
    default: return go_v1<PAIR, XK, 16>(o, tiles, s);
    }
}

// Launches the problems of one input kind: one activation row (the norm
// kinds always) -> the one-row kernel; up to four rows -> the MFMA kernel.
// PAIR only comes with the norm, as in the fused chain.
hipError_t launch_lds_kind(GemvBatch &b, int xk, hipStream_t s) {
    const bool pair = b.p[0].pair != 0;
    switch (xk) {
    case kXkNorm | kXkM1: return pair ? launch_v1<true, kXkNorm>(b, s) : launch_v1<false, kXkNorm>(b, s);
    case kXkF32 | kXkNorm | kXkM1:
        return pair ? launch_v1<true, kXkF32 | kXkNorm>(b, s) : launch_v1<false, kXkF32 | kXkNorm>(b, s);
    case kXkM1: return pair ? hipErrorInvalidValue : launch_v1<false, kXkM1>(b, s);
    case kXkF32 | kXkM1: return pair ? hipErrorInvalidValue : launch_v1<false, kXkF32 | kXkM1>(b, s);
    case 0: return pair ? hipErrorInvalidValue : launch_lds<false, 0>(b, s);
    case kXkF32: return pair ? hipErrorInvalidValue : launch_lds<false, kXkF32>(b, s);
    default: return hipErrorInvalidValue;
    }
}

hipError_t launch_gemv_batch(GemvBatch &b, hipStream_t s) {
    if (b.p[0].mode != 0) {
        bool ok = true;
        for (int i = 0; i < b.n; ++i) {
            const GemvProblem &p = b.p[i];
            const int per = x_per_chunk(p.x_dt);
            const int E = x_chunks(p.K, p.x_dt, kQuantLanes);
            if (p.mode == 0 || (p.x_dt != BL_BF16 && p.x_dt != BL_F32) || p.M > kFuseMaxM || p.M * E > kXRegs ||
                (p.mode == 2 && (p.M != 1 || E * per / 4 > kXRegs)) ||
                (size_t)p.M * ((p.K + kUnitK - 1) / kUnitK * kUnitK) > (size_t)kLdsQBytes ||
                ((uintptr_t)p.gain % 16) != 0 || p.K % 16 != 0 || p.K % per != 0 || p.ldx % per != 0 ||
                (p.pair != 0) != (b.p[0].pair != 0) || (p.pair != 0 && p.mode != 2))
                ok = false;
        }
        if (ok) {
            // one launch per input kind present (output rows are disjoint)
            bool done[kMaxProblems] = {};
            for (int i = 0; i < b.n; ++i) {
                if (done[i]) continue;
                const int xk = xkind_of(b.p[i]);
                GemvBatch g;
                memset(&g, 0, sizeof(g));
                for (int j = i; j < b.n; ++j)
                    if (!done[j] && xkind_of(b.p[j]) == xk) {
                        g.p[g.n++] = b.p[j];
                        done[j] = true;
                    }
                if (hipError_t e = launch_lds_kind(g, xk, s); e != hipSuccess) return e;
            }
            return hipSuccess;
        }
    }
    bool tiled = false;
    for (int i = 0; i < b.n; ++i) tiled = tiled || b.p[i].qtile != 0;
    if (tiled) {
        // tiled codes are read by k_gemv_mt only
        if (!gemv_mt_ok(b)) return hipErrorInvalidValue;
        const hipError_t e = launch_gemv_mt(b, s);
        return e == hipErrorNotSupported ? hipErrorInvalidValue : e;
    }
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

hipError_t gemv_wait_expired(unsigned int *count, bool reset) {
    unsigned int v = 0;
    if (hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_wait_expired), sizeof(v)); e != hipSuccess) return e;
    if (reset && v) {
        const unsigned int zero = 0;
        if (hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_wait_expired), &zero, sizeof(zero)); e != hipSuccess)
            return e;
    }
    *count = v;
    return hipSuccess;
}

} // namespace bl
