// k_contract.hip -- the int8 x ternary contraction with its rescale epilogue.
//
// "Transformers 实战 BitNet 1.58 位量化", section "推理侧 BitLinear：打包权重、解包与缩放":
// the inference forward multiplies the int8 activations with the unpacked
// ternary weight and rescales the product by the activation and weight
// scales; the unpack reads field i of a packed byte under the mask 3 << 2i
// and subtracts 1.  Here the weights are never unpacked to memory: every
// kernel expands the 2-bit fields in registers and feeds them to the gfx950
// int8 matrix cores (v_mfma_i32_16x16x64_i8).
//
// Expansion without the -1: for a packed dword b (four k's of one packed
// row), b & 0x03030303, b & 0x0C0C0C0C, b & 0x30303030 and (b >> 2) &
// 0x30303030 are four int8x4 operands holding v*1, v*4, v*16, v*16 with
// v = code + 1 in {0,1,2} for fields 0..3.  The matrix core accumulates
// sum_k q*v scaled by that power of two; an exact arithmetic shift undoes it,
// and subtracting sum_k q (the row sum of the codes over the same k range)
// gives the exact sum_k q*code.  With |q| <= 128 and K < 2^19 every partial
// stays inside int32.
//
// MFMA operand layout used (16x16x64, int8): lane l supplies row (l & 15) of
// A and column (l & 15) of B, each as 16 int8 values of k-group (l >> 4);
// A and B use the same k placement, so any consistent assignment of k to
// (group, byte) gives the same dot products.  The 16x16 int32 result sits in
// lane l as rows 4*(l >> 4) + j, column l & 15, for j = 0..3.
#include "bl_common.h"

namespace bl {

namespace {

typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i ld16(const void *p) {
    return *reinterpret_cast<const v4i *>(p);
}

__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

// Field operands of 16 packed bytes (see the header comment).
__device__ __forceinline__ void expand(v4i b, v4i f[4]) {
    f[0] = b & 0x03030303;
    f[1] = b & 0x0C0C0C0C;
    f[2] = b & 0x30303030;
    f[3] = (b >> 2) & 0x30303030;
}


__device__ __forceinline__ int rowsum16(v4i a) {
    int s = __builtin_amdgcn_sdot4(a.x, 0x01010101, 0, false);
    s = __builtin_amdgcn_sdot4(a.y, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(a.z, 0x01010101, s, false);
    s = __builtin_amdgcn_sdot4(a.w, 0x01010101, s, false);
    return s;
}

__device__ __forceinline__ int shift_field(int v, int f) {
    return f == 0 ? v : (f == 1 ? (v >> 2) : (v >> 4));
}

// Final output of one accumulator entry.
__device__ __forceinline__ void emit(const Contract &c, int m, int vr, int f, int A, int U) {
    const float a = c.a[m];
    if (c.pair) {
        const int col = f * c.R + vr;
        const float gv = (float)A * (c.w_mean[0] / a);
        const float uv = (float)U * (c.w_mean[1] / a);
        const float p = relu2_mul(gv, uv);
        const size_t idx = (size_t)m * c.ldy + col;
        if (c.y_dt == BL_BF16)
            ((uint16_t *)c.y)[idx] = f32_to_bf16(p);
        else
            ((float *)c.y)[idx] = p;
    } else {
        const ColOf cs = col_of(c.seg, vr, f);
        const float scale = c.w_mean[cs.seg] / a;
        store_out(c.y, c.y_dt, (size_t)m * c.ldy + cs.col, A, scale);
    }
}

// ===========================================================================
// Decode kernel (M <= 64).
// One workgroup = 8 waves on one tile of 16 packed rows (64 output columns;
// PAIR: 16 gate rows and the 16 matching up rows).  The workgroup owns a
// range of 64-wide k-steps; wave w takes steps base + w + 8s (s < KS), so at
// any moment the 8 waves read 8 adjacent 64-byte pieces of the same 16 rows.
// Packed bytes go straight from HBM to registers (each byte is used once);
// activation codes are small and come from L2.  Partial sums are reduced
// across the 8 waves with LDS integer atomics.  When one tile is split over
// several workgroups (nchunks > 1), those add their partials into an int32
// scratch with device-scope atomics, and the last one to arrive (ticket)
// reads them back, clears them, and writes the outputs.
// ===========================================================================
constexpr int kGemvWaves = 8;

template <int MT, int KS, bool PAIR>
__global__ __launch_bounds__(kGemvWaves * 64) void k_gemv(Contract c, int32_t *__restrict__ acc,
                                                          unsigned *__restrict__ tickets,
                                                          int nchunks, int ldacc) {
    constexpr int NB = PAIR ? 2 : 1;                  // weight rows per lane
    constexpr int NE = MT * 4 * 4 * 64;               // accumulator entries per tensor
    __shared__ int red[NB][NE];

    const int wave = threadIdx.x >> 6;
    const int lane = threadIdx.x & 63;
    const int lr = lane & 15;
    const int g = lane >> 4;
    const int tile = blockIdx.x / nchunks;
    const int chunk = blockIdx.x - tile * nchunks;
    const int r0 = tile * 16;
    const int vr = r0 + lr;
    const bool row_ok = vr < c.R;
    const int K = c.K;
    const int nsteps = (K + 63) >> 6;
    const int base = chunk * (kGemvWaves * KS);

    for (int i = threadIdx.x; i < NB * NE; i += kGemvWaves * 64) (&red[0][0])[i] = 0;

    const uint8_t *pw[NB];
    pw[0] = c.P + (size_t)vr * K + 16 * g;
    if (PAIR) pw[NB - 1] = c.P + (size_t)(c.R + vr) * K + 16 * g;

    // Issue every load of this wave before any use.
    v4i bv[NB][KS];
    v4i av[MT][KS];
#pragma unroll
    for (int s = 0; s < KS; ++s) {
        const int st = base + wave + kGemvWaves * s;
        const int kk = st * 64 + 16 * g;
        const bool kok = st < nsteps && kk < K;
#pragma unroll
        for (int t = 0; t < NB; ++t)
            bv[t][s] = (kok && row_ok) ? ld16(pw[t] + st * 64) : v4i{0, 0, 0, 0};
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) {
            const int m = mt * 16 + lr;
            av[mt][s] = (kok && m < c.M) ? ld16(c.q + (size_t)m * c.ldq + kk) : v4i{0, 0, 0, 0};
        }
    }

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

#pragma unroll
    for (int s = 0; s < KS; ++s) {
#pragma unroll
        for (int mt = 0; mt < MT; ++mt) qs[mt] += rowsum16(av[mt][s]);
#pragma unroll
        for (int t = 0; t < NB; ++t) {
            v4i fb[4];
            expand(bv[t][s], fb);
#pragma unroll
            for (int mt = 0; mt < MT; ++mt)
#pragma unroll
                for (int f = 0; f < 4; ++f) accv[t][mt][f] = mfma16(av[mt][s], fb[f], accv[t][mt][f]);
        }
    }

    // Row sums over this wave's k range: reduce the four k-groups.
#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
        qs[mt] += __shfl_xor(qs[mt], 16, 64);
        qs[mt] += __shfl_xor(qs[mt], 32, 64);
    }
    __syncthreads();   // LDS cleared

#pragma unroll
    for (int mt = 0; mt < MT; ++mt) {
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int qsum = __shfl(qs[mt], 4 * g + j, 64);
            if (mt * 16 + 4 * g + j >= c.M) continue;
#pragma unroll
            for (int t = 0; t < NB; ++t)
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int v = shift_field(accv[t][mt][f][j], f) - qsum;
                    atomicAdd(&red[t][((mt * 4 + f) * 4 + j) * 64 + lane], v);
                }
        }
    }
    __syncthreads();

    // Entries: e -> (mt, f, j, lane) with the layout used above.
    auto entry_mvr = [&](int e, int &m, int &vrr, int &f) {
        const int ln = e & 63;
        const int j = (e >> 6) & 3;
        f = (e >> 8) & 3;
        const int mt = e >> 10;
        m = mt * 16 + 4 * (ln >> 4) + j;
        vrr = r0 + (ln & 15);
    };
    auto acc_index = [&](int m, int vrr, int f, int t) -> size_t {
        int col;
        if (PAIR) col = t * 4 * c.R + f * c.R + vrr;
        else col = col_of(c.seg, vrr, f).col;
        return (size_t)m * ldacc + col;
    };

    if (nchunks == 1) {
        for (int e = threadIdx.x; e < NE; e += kGemvWaves * 64) {
            int m, vrr, f;
            entry_mvr(e, m, vrr, f);
            if (m >= c.M || vrr >= c.R) continue;
            emit(c, m, vrr, f, red[0][e], PAIR ? red[NB - 1][e] : 0);
        }
        return;
    }

    for (int e = threadIdx.x; e < NE; e += kGemvWaves * 64) {
        int m, vrr, f;
        entry_mvr(e, m, vrr, f);
        if (m >= c.M || vrr >= c.R) continue;
#pragma unroll
        for (int t = 0; t < NB; ++t) atomicAdd(&acc[acc_index(m, vrr, f, t)], red[t][e]);
    }
    __threadfence();
    __syncthreads();
    __shared__ int last;
    if (threadIdx.x == 0) last = (atomicAdd(&tickets[tile], 1u) == (unsigned)(nchunks - 1));
    __syncthreads();
    if (!last) return;
    __threadfence();
    for (int e = threadIdx.x; e < NE; e += kGemvWaves * 64) {
        int m, vrr, f;
        entry_mvr(e, m, vrr, f);
        if (m >= c.M || vrr >= c.R) continue;
        const int A = atomicExch(&acc[acc_index(m, vrr, f, 0)], 0);
        const int U = PAIR ? atomicExch(&acc[acc_index(m, vrr, f, NB - 1)], 0) : 0;
        emit(c, m, vrr, f, A, U);
    }
    if (threadIdx.x == 0) atomicExch(&tickets[tile], 0u);
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

// ---------------------------------------------------------------------------
// Host-side dispatch
// ---------------------------------------------------------------------------
template <int MT, int KS, bool PAIR>
hipError_t gemv_launch(const Contract &c, int32_t *acc, unsigned *tickets, int ntiles, int nchunks,
                       int ldacc, hipStream_t s) {
    hipLaunchKernelGGL((k_gemv<MT, KS, PAIR>), dim3(ntiles * nchunks), dim3(kGemvWaves * 64), 0, s, c,
                       acc, tickets, nchunks, ldacc);
    return hipGetLastError();
}

template <int MT, bool PAIR>
hipError_t gemv_ks(int KS, const Contract &c, int32_t *acc, unsigned *tickets, int ntiles,
                   int nchunks, int ldacc, hipStream_t s) {
    switch (KS) {
    case 1: return gemv_launch<MT, 1, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 2: return gemv_launch<MT, 2, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 3: return gemv_launch<MT, 3, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 4: return gemv_launch<MT, 4, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 5: return gemv_launch<MT, 5, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 6: return gemv_launch<MT, 6, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    default: return gemv_launch<MT, 8, PAIR>(c, acc, tickets, ntiles, nchunks, ldacc, s);
    }
}

template <bool PAIR>
hipError_t gemv_mt(int MT, int KS, const Contract &c, int32_t *acc, unsigned *tickets, int ntiles,
                   int nchunks, int ldacc, hipStream_t s) {
    switch (MT) {
    case 1: return gemv_ks<1, PAIR>(KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 2: return gemv_ks<2, PAIR>(KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
    case 3: return gemv_ks<3, PAIR>(KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
    default: return gemv_ks<4, PAIR>(KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
    }
}

} // namespace

// Work split of the decode kernel: steps per wave (KS) and workgroups per
// tile (nchunks).  Aim for at least ~2048 waves in flight (8 per CU) while
// keeping at least 3/4 of the wave-steps busy; split a tile across
// workgroups only when the int32 scratch can hold the outputs.
void gemv_plan(int M, int R, int K, bool pair, bool can_split, int &KS, int &nchunks) {
    const int nsteps = (K + 63) / 64;
    const int ntiles = (R + 15) / 16;
    const int target = M > 16 ? 1024 : 2048;
    static const int cand[] = {8, 6, 5, 4, 3, 2, 1};
    // register budget: the widest variants (4 token tiles, gate and up) spill above 4 steps
    const int ks_max = ((M + 15) / 16) * (pair ? 2 : 1) >= 6 ? 4 : 8;
    KS = 1;
    nchunks = (nsteps + kGemvWaves - 1) / kGemvWaves;
    bool found = false;
    for (int ks : cand) {
        if (ks > ks_max) continue;
        const int spw = kGemvWaves * ks;
        const int nch = (nsteps + spw - 1) / spw;
        if (nch > 1 && !can_split) continue;
        const double util = (double)nsteps / (double)(nch * spw);
        if (util < 0.75) continue;
        if ((int64_t)ntiles * nch * kGemvWaves >= target) {
            KS = ks;
            nchunks = nch;
            found = true;
            break;
        }
    }
    if (!found) {
        if (can_split) {
            KS = 1;
            nchunks = (nsteps + kGemvWaves - 1) / kGemvWaves;
        } else {
            // one workgroup per tile: smallest KS covering all steps
            for (int ks : {1, 2, 3, 4, 5, 6, 8}) {
                if (ks > ks_max) break;
                KS = ks;
                if (kGemvWaves * ks >= nsteps) break;
            }
            nchunks = (nsteps + kGemvWaves * KS - 1) / (kGemvWaves * KS);
        }
    }
}

hipError_t launch_gemv(const Contract &c, int32_t *acc, size_t acc_cap, unsigned *tickets,
                       int ticket_cap, hipStream_t s) {
    const int ntiles = (c.R + 15) / 16;
    const int ldacc = c.pair ? 8 * c.R : 4 * c.R;
    const bool can_split = acc != nullptr && tickets != nullptr && ntiles <= ticket_cap &&
                           (size_t)c.M * ldacc * sizeof(int32_t) <= acc_cap;
    int KS, nchunks;
    gemv_plan(c.M, c.R, c.K, c.pair, can_split, KS, nchunks);
    const int MT = (c.M + 15) / 16;
    if (c.pair) return gemv_mt<true>(MT, KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
    return gemv_mt<false>(MT, KS, c, acc, tickets, ntiles, nchunks, ldacc, s);
}

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
