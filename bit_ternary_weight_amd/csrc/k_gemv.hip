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

// ===========================================================================
// Streaming variant for the fused path (M <= 4): the packed weights land in
// LDS through the gfx950 direct global->LDS loads (global_load_lds_dwordx4),
// so the bytes in flight cost no registers and two workgroups share a CU.
// Each wave owns a ring of RING 1 KB slots per weight tensor; lane l's 16
// bytes of a k-step land at slot + 16*l and only lane l reads them back, so a
// wave needs no barrier to consume its own slots: it waits for its oldest
// load (s_waitcnt vmcnt), reads the slot, and immediately refills it with the
// step RING places ahead.  The raw activation rows are loaded into registers
// before any weight load, so the quantization prologue (which needs only
// them) never waits behind the weight stream.
// ===========================================================================
constexpr int kRing = 7;
constexpr int kLdsWaves = 8;
constexpr int kLdsQBytes = 8192;   // static LDS for the activation codes (M*K)
constexpr int kXChunks = 4;   // 16-byte activation chunks per lane (all rows); row_pass selects among 4

// Activation elements per 16-byte chunk.
__host__ __device__ constexpr int x_per_chunk(int dt) { return dt == BL_BF16 ? 8 : 4; }

// Chunks per row for K elements (every lane takes chunk c at element
// (c * lanes + lane) * per_chunk).
__host__ __device__ inline int x_chunks(int K, int dt, int lanes) {
    const int per = x_per_chunk(dt) * lanes;
    return (K + per - 1) / per;
}

// Workgroup barrier ordering LDS only: wait for this wave's LDS operations
// (lgkmcnt 0), then s_barrier.  __syncthreads() (and the compiler's own
// barrier lowering) would also wait for every outstanding global load of the
// wave, i.e. for the whole weight stream in flight.  The barrier is written
// as an asm statement with a memory clobber so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
}

template <int W>
__device__ __forceinline__ float block_max_lds(float v, float *rf) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) rf[threadIdx.x >> 6] = v;
    lds_barrier();
    float r = rf[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r = fmaxf(r, rf[i]);
    lds_barrier();
    return r;
}

template <int W>
__device__ __forceinline__ double block_sum_lds(double v, double *rd) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) rd[threadIdx.x >> 6] = v;
    lds_barrier();
    double r = rd[0];
#pragma unroll
    for (int i = 1; i < W; ++i) r += rd[i];
    lds_barrier();
    return r;
}

// Element i of a 16-byte activation chunk (static i after unrolling).
template <int PER>
__device__ __forceinline__ float chunk_elem(const v4i &c, int i) {
    if (PER == 8) {
        const uint32_t w = (uint32_t)c[i >> 1];
        return __uint_as_float((i & 1) ? (w & 0xFFFF0000u) : (w << 16));
    }
    return __uint_as_float((uint32_t)c[i]);
}

// One pass of the prologue over the register chunks of row m:
// OP 0 accumulates sum v^2 (fp64), OP 1 the max |v|, OP 2 quantizes into q_s.
// Register j of an array of four, with static indices only (a dynamic index
// would put the array in scratch memory).
__device__ __forceinline__ v4i pick4(const v4i *a, int j) {
    return j == 0 ? a[0] : (j == 1 ? a[1] : (j == 2 ? a[2] : a[3]));
}

template <int PER, int OP>
__device__ __forceinline__ void row_pass(const GemvProblem &p, const v4i *xr, const v4i *gr, int E, int m,
                                         int lanes, float r, float s, bool norm, int8_t *q_s, double &ss,
                                         float &amax) {
    const int K = p.K;
    // fully unrolled (static bounds, predicated): a loop reading registers
    // loaded before it would make the compiler wait for every load in flight
#pragma unroll
    for (int c = 0; c < kXChunks; ++c) {
        const int k0 = (c * lanes + (int)threadIdx.x) * PER;
        if (c >= E || k0 >= K) continue;   // K % PER == 0: a chunk is all in or all out
        const v4i xc = pick4(xr, m * E + c);
        // gains of this chunk: PER floats = PER/4 registers starting at gr[c*PER/4]
        const v4i g0 = pick4(gr, c * (PER / 4));
        const v4i g1 = PER == 8 ? pick4(gr, c * 2 + 1) : g0;
        uint32_t pk[2] = {0, 0};
#pragma unroll
        for (int i = 0; i < PER; ++i) {
            float t = chunk_elem<PER>(xc, i);
            if (OP == 0) {
                ss += (double)t * (double)t;
                continue;
            }
            if (norm) {
                t = t * r;
                if (p.gain) t = t * __uint_as_float((uint32_t)(i < 4 ? g0[i & 3] : g1[i & 3]));
            }
            if (OP == 1) amax = fmaxf(amax, fabsf(t));
            else pk[i >> 2] |= (uint32_t)(quant1(t, s) & 0xFF) << (8 * (i & 3));
        }
        if (OP == 2) {
            int8_t *dst = q_s + (size_t)m * K + k0;
            if (PER == 8) *reinterpret_cast<uint2 *>(dst) = make_uint2(pk[0], pk[1]);
            else *reinterpret_cast<uint32_t *>(dst) = pk[0];
        }
    }
}

// Quantize the M (<= 4) rows held in xr (row m, chunk c at xr[m*E + c]) into
// q_s and a_s; same arithmetic as prologue().  Global memory is not touched
// (no loads or stores may sit between the weight loads in flight).
template <int W, int PER>
__device__ void prologue_regs(const GemvProblem &p, const v4i *xr, const v4i *gr, int E, int8_t *q_s, float *a_s,
                              double *rd, float *rf) {
    const bool norm = p.mode == 2;
    const int lanes = W * 64;
#pragma unroll
    for (int m = 0; m < kFuseMaxM; ++m) {
        if (m >= p.M) break;
        double ss = 0.0;
        float amax = 0.0f;
        float r = 1.0f;
        if (norm) {
            row_pass<PER, 0>(p, xr, gr, E, m, lanes, 1.0f, 0.0f, norm, q_s, ss, amax);
            ss = block_sum_lds<W>(ss, rd);
            r = (float)(1.0 / sqrt(ss / (double)p.K + (double)p.eps));
        }
        row_pass<PER, 1>(p, xr, gr, E, m, lanes, r, 0.0f, norm, q_s, ss, amax);
        amax = block_max_lds<W>(amax, rf);
        const float s = 127.0f / fmaxf(amax, kFloor);   // IEEE fp32 division
        if (threadIdx.x == 0) a_s[m] = s;
        row_pass<PER, 2>(p, xr, gr, E, m, lanes, r, s, norm, q_s, ss, amax);
    }
}

// s_waitcnt immediate (gfx9 encoding) for vmcnt = VM, leaving expcnt and
// lgkmcnt unconstrained: vmcnt[3:0] | expcnt[6:4] | lgkmcnt[11:8] | vmcnt[15:14].
template <int VM>
struct kWaitVm {
    static_assert(VM >= 0 && VM < 64, "vmcnt is 6 bits");
    static constexpr int value = (VM & 0xF) | (0x7 << 4) | (0xF << 8) | ((VM >> 4) << 14);
};

// s_waitcnt vmcnt(n) for a run-time n in [0, 2*kRing] (the counter field is an
// immediate, so dispatch over the possible values).
__device__ __forceinline__ void wait_vm(int n) {
    switch (n) {
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
    case 12: __builtin_amdgcn_s_waitcnt(kWaitVm<12>::value); break;
    case 13: __builtin_amdgcn_s_waitcnt(kWaitVm<13>::value); break;
    default: __builtin_amdgcn_s_waitcnt(kWaitVm<14>::value); break;
    }
}

__device__ __forceinline__ void dma16(const void *src, void *lds_slot) {
    __builtin_amdgcn_global_load_lds(src, lds_slot, 16, 0, 0);
}

// Occupancy target: two 8-wave workgroups per CU (4 waves per SIMD, <= 128
// VGPRs); the LDS ring (kRing KB per wave and tensor) bounds it as well.
template <bool PAIR>
__global__ __launch_bounds__(kLdsWaves * 64) __attribute__((amdgpu_waves_per_eu(4, 4)))
void k_gemv_lds(GemvBatch b) {
    constexpr int W = kLdsWaves;
    constexpr int NB = PAIR ? 2 : 1;
    constexpr int NE = 1024;   // MT == 1
    // Static LDS objects (distinct from the dynamic weight ring, so the
    // compiler can tell that writing them does not race the ring's loads);
    // the dynamic ring then starts after them, never at LDS address 0.
    __shared__ int red[NB * NE];
    __shared__ float a_s[64];
    __shared__ double rd[16];
    __shared__ float rf[16];
    __shared__ __attribute__((aligned(16))) int8_t q_s[kLdsQBytes];
    __shared__ float wm_s[BL_MAX_SEGMENTS];
    extern __shared__ __attribute__((aligned(16))) unsigned char ring_lds[];

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
    const int ks = (nsteps + W - 1) / W;   // steps of this wave: wave + W*i, i < ks
    unsigned char *ring = ring_lds + (size_t)wave * (kRing * NB * 1024);

    // 1. the raw activation rows, into registers, before any weight load
    const int E = x_chunks(K, p.x_dt, W * 64);
    v4i xr[kXChunks];
    v4i gr[kXChunks];
    {
        const int per = x_per_chunk(p.x_dt);
        const int esz = p.x_dt == BL_BF16 ? 2 : 4;
        // unconditional loads (out-of-range chunks read row 0, chunk 0 and are
        // never used), so the wait counter sees straight-line code
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int m = j / (E > 0 ? E : 1);
            const int c = j - m * E;
            const int k0 = (c * W * 64 + (int)threadIdx.x) * per;
            const bool ok = j < M * E && k0 < K;
            xr[j] = ld16((const unsigned char *)p.x + (ok ? ((size_t)m * p.ldx + k0) * esz : 0));
        }
        // RMSNorm gains of this lane's chunks (shared by the rows): register
        // c*per/4 + h holds gain[k0(c) + 4h .. +3]; unused ones read x.
#pragma unroll
        for (int j = 0; j < kXChunks; ++j) {
            const int c = j / (per / 4);
            const int h = j - c * (per / 4);
            const int k0 = (c * W * 64 + (int)threadIdx.x) * per + 4 * h;
            const bool ok = p.gain != nullptr && p.mode == 2 && c < E && k0 < K;
            gr[j] = ok ? ld16(p.gain + k0) : ld16(p.x);
        }
    }

    // the weight scales of the output segments, with the same early loads
    const int nscale = PAIR ? 2 : p.seg.n;
    const float wmv = (int)threadIdx.x < nscale ? p.w_mean[threadIdx.x] : 0.0f;

    // Every wave issues its activation loads before any wave issues a weight
    // load (the CU's memory pipeline is shared: a wave's activation loads
    // must not queue behind the other waves' weight stream).
    lds_barrier();

    // 2. fill the ring with this wave's first min(ks, kRing) steps.  Every
    // lane of a wave issues each load (lanes outside the tile or past K read
    // a fixed valid address; their slot bytes are masked on use), so the
    // wave's outstanding-load count is known exactly at every wait below.
    const uint8_t *pw[NB];
    pw[0] = p.P + (size_t)vr * K + 16 * g;
    if (PAIR) pw[NB - 1] = p.P + (size_t)(p.R + vr) * K + 16 * g;
    auto src_of = [&](int t, int i) -> const void * {
        const int st = wave + W * i;
        const bool ok = i < ks && st * 64 + 16 * g < K && row_ok;
        return ok ? (const void *)(pw[t] + st * 64) : (const void *)p.P;
    };
    // The prefill is always kRing steps (steps past this wave's last read the
    // fixed address), so the wait below has a constant count.
#pragma unroll
    for (int i = 0; i < kRing; ++i)
#pragma unroll
        for (int t = 0; t < NB; ++t) dma16(src_of(t, i), ring + (i * NB + t) * 1024);

    // The activation, gain and scale loads are older than the kRing*NB weight
    // loads just issued: this wait retires them without waiting for any of those.
    __builtin_amdgcn_s_waitcnt(kWaitVm<kRing * NB>::value);
    if ((int)threadIdx.x < nscale) wm_s[threadIdx.x] = wmv;

    // 3. prologue: quantize the activation rows into LDS (uses only xr)
    for (int i = threadIdx.x; i < NB * NE; i += W * 64) red[i] = 0;
    if (p.x_dt == BL_BF16) prologue_regs<W, 8>(p, xr, gr, E, q_s, a_s, rd, rf);
    else prologue_regs<W, 4>(p, xr, gr, E, q_s, a_s, rd, rf);
    lds_barrier();

    // 4. stream: consume step i from its slot, refill the slot with step i + kRing
    v4i accv[NB][4];
#pragma unroll
    for (int t = 0; t < NB; ++t)
#pragma unroll
        for (int f = 0; f < 4; ++f) accv[t][f] = v4i{0, 0, 0, 0};
    int qs = 0;
    for (int i = 0; i < ks; ++i) {
        const int slot = i % kRing;
        const int st = wave + W * i;
        const int kk = st * 64 + 16 * g;
        const bool kok = kk < K;
        // slots issued so far: the kRing prefill plus one refill per earlier
        // iteration that had a step kRing ahead; all issued after step i may
        // stay outstanding
        const int issued = kRing + (i < ks - kRing ? i : (ks > kRing ? ks - kRing : 0));
        wait_vm((issued - i - 1) * NB);
        v4i bw[NB];
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            bw[t] = *reinterpret_cast<const v4i *>(ring + (slot * NB + t) * 1024 + 16 * lane);
            if (!(kok && row_ok)) bw[t] = v4i{0, 0, 0, 0};
        }
        // refill the slot with step i + kRing when this wave has one
        if (i + kRing < ks) {
#pragma unroll
            for (int t = 0; t < NB; ++t) dma16(src_of(t, i + kRing), ring + (slot * NB + t) * 1024);
        }
        const v4i a_op = (kok && lr < M) ? *reinterpret_cast<const v4i *>(q_s + (size_t)lr * K + kk)
                                         : v4i{0, 0, 0, 0};
        qs += rowsum16(a_op);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            v4i fb[4];
            expand(bw[t], fb);
#pragma unroll
            for (int f = 0; f < 4; ++f) accv[t][f] = mfma16(a_op, fb[f], accv[t][f]);
        }
    }

    // No weight load may still be writing LDS once the workgroup ends (its
    // LDS can be handed to the next workgroup): drain the ring.
    __builtin_amdgcn_s_waitcnt(kWaitVm<0>::value);

    // The first tile's workgroup hands out its activation codes and scales
    // (stage outputs for checks), now that no weight load is in flight.
    if (tile == 0 && p.dbg_q != nullptr) {
        for (int i = threadIdx.x; i < M * K; i += W * 64) p.dbg_q[i] = q_s[i];
        if (p.dbg_a != nullptr && (int)threadIdx.x < M) p.dbg_a[threadIdx.x] = a_s[threadIdx.x];
    }

    // 5. reduce across waves, rescale, store
    qs += __shfl_xor(qs, 16, 64);
    qs += __shfl_xor(qs, 32, 64);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int qsum = __shfl(qs, 4 * g + j, 64);
        if (4 * g + j >= M) continue;
#pragma unroll
        for (int t = 0; t < NB; ++t)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int v = shift_field(accv[t][f][j], f) - qsum;
                atomicAdd(&red[t * NE + (f * 4 + j) * 64 + lane], v);
            }
    }
    lds_barrier();
    for (int e = threadIdx.x; e < NE; e += W * 64) {
        const int ln = e & 63;
        const int j = (e >> 6) & 3;
        const int f = (e >> 8) & 3;
        const int m = 4 * (ln >> 4) + j;
        const int vrr = r0 + (ln & 15);
        if (m >= M || vrr >= p.R) continue;
        emit_out(p.y, p.y_dt, p.ldy, PAIR, p.seg, p.R, wm_s, m, vrr, f, a_s[m], red[e],
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

// Streaming variant (fused path, every problem's rows in kXChunks register
// chunks): problems ordered by decreasing K so the longest tiles start first.
template <bool PAIR>
hipError_t launch_lds(GemvBatch &b, hipStream_t s) {
    constexpr int NB = PAIR ? 2 : 1;
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
        o.p[i] = b.p[order[i]];
        o.p[i].tile0 = tiles;
        tiles += (o.p[i].R + 15) / 16;
    }
    o.ring_off = 0;
    const size_t lds = (size_t)kLdsWaves * kRing * NB * 1024;   // dynamic part: the weight ring
    // Dynamic LDS above the default 64 KiB must be allowed per kernel (the
    // static part, at most ~17 KiB, comes on top; both fit the 160 KiB).
    static size_t attr_bytes = 0;
    if (attr_bytes < lds) {
        hipError_t e = hipFuncSetAttribute((const void *)k_gemv_lds<PAIR>,
                                           hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
        if (e != hipSuccess) {
            (void)hipGetLastError();   // do not leave the error to the next launch
            return e;
        }
        attr_bytes = lds;
    }
    hipLaunchKernelGGL(k_gemv_lds<PAIR>, dim3(tiles), dim3(kLdsWaves * 64), lds, s, o);
    return hipGetLastError();
}

hipError_t launch_gemv_batch(GemvBatch &b, hipStream_t s) {
    if (b.p[0].mode != 0) {
        bool ok = true;
        for (int i = 0; i < b.n; ++i) {
            const GemvProblem &p = b.p[i];
            const int per = x_per_chunk(p.x_dt);
            if (p.mode == 0 || p.M > kFuseMaxM || p.M * x_chunks(p.K, p.x_dt, kLdsWaves * 64) > kXChunks ||
                (size_t)p.M * p.K > (size_t)kLdsQBytes || ((uintptr_t)p.gain % 16) != 0 ||
                p.K % per != 0 || p.ldx % per != 0 || (p.pair != 0) != (b.p[0].pair != 0))
                ok = false;
        }
        if (ok) return b.p[0].pair ? launch_lds<true>(b, s) : launch_lds<false>(b, s);
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

} // namespace bl
