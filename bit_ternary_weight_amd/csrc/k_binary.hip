// k_binary.hip -- the 1-bit BitLinear: layer normalization, sign-binarized
// weights (one bit each, one scale per tensor), absmax int8 activations and
// the int8 x 1-bit contraction on the matrix cores.
//
// The PyTorch 1-bit BitNet project summary, section "How It Works": the
// BitLinear that replaces a linear layer binarizes its weights and feeds it
// activations that went through layer normalization and absolute-maximum
// quantization.  The page prints no formula; the readings (shared with the
// oracle, written independently there):
//   * sign: -1 where W < 0, else +1; scale: the mean of |W| (the ternary
//     path's absmean kernels: fp64 sum, fp32, floor 1e-5);
//   * bit i of packed row r (plane order, N/8 packed rows) is weight row
//     i*N/8 + r, set for +1;
//   * mu and the variance in fp64, r = float(1/sqrt(var + eps)),
//     x' = (float(x - mu) * r) * gamma + beta, then the ternary path's
//     absmax int8 quantization, y = float(A) * (w_scale / a).
//
// The contraction: for a packed dword b (four k's of one packed row), the
// int8x4 operand b & (0x01010101 << i) holds bit_i * 2^i for i = 0..6, and
// (b >> 1) & 0x40404040 holds bit_7 * 64; the matrix core sums q * that, an
// exact shift removes the power of two, and A = 2 sum_k q*bit - sum_k q
// turns {0,1} into {-1,+1}.  |A| <= 64 * 128 * K stays inside int32 for
// K <= 16384.
#include "bl_common.h"

#include <utility>

namespace bl {

namespace {

constexpr int kT = 256;
constexpr int kLnMaxChunks = 16;   // float4 chunks per thread in the norm: K <= 16384

struct W1Problem {
    const void *x;        // raw activations [M, ldx] (layer-norm launch), or null
    int x_dt, ldx;
    const float *gamma;   // [K] or null
    const float *beta;    // [K] or null
    int M, K;
    int8_t *q;            // [M, K] codes
    float *a;             // [M] activation scales
    const uint8_t *P;     // packed signs [N/8, K]
    int N;
    const float *w_scale; // [1]
    float *y;             // [M, N]
};

struct W1Batch {
    W1Problem p[kMaxProblems];
    int n;
    int start[kMaxProblems + 1];   // first workgroup of each problem
    int quads[kMaxProblems];       // single-token launch: row quads (4 packed rows) per workgroup, 1, 2 or 4
    float eps;
};

// The launch's single argument, read through the kernel-argument pointer so
// that a run-time problem index is a scalar load, not a copy of the table.
__device__ __forceinline__ const W1Batch &batch() {
    return *(const W1Batch *)__builtin_amdgcn_kernarg_segment_ptr();
}

// Problem of this workgroup and the workgroup's index within it (and, when
// asked, the problem's row quads per workgroup).  The loop has a fixed trip
// count and carries the selected values along, so all its kernel-argument
// loads go out together: a loop bounded by b.n, with b.start[p] read after
// it, compiled to one dependent round trip per problem.
__device__ __forceinline__ int problem_of(const W1Batch &b, int &local, int *quads = nullptr) {
    const int blk = blockIdx.x;
    int p = 0, st = b.start[0], qd = b.quads[0];
#pragma unroll
    for (int i = 1; i < kMaxProblems; ++i) {
        const bool in = i < b.n && blk >= b.start[i];   // selects, no branch around the loads
        p = in ? i : p;
        st = in ? b.start[i] : st;
        qd = in ? b.quads[i] : qd;
    }
    local = blk - st;
    if (quads) *quads = qd;
    return p;
}

// ---------------------------------------------------------------------------
// Packing: one lane per 4 consecutive k of one packed row (K % 4 == 0).
// ---------------------------------------------------------------------------
__global__ __launch_bounds__(kT) void k_binarize_pack4(const float *__restrict__ W, int N, int K,
                                                       uint8_t *__restrict__ P) {
    const int R = N / 8, K4 = K / 4;
    const int64_t idx = (int64_t)blockIdx.x * kT + threadIdx.x;
    if (idx >= (int64_t)R * K4) return;
    const int r = (int)(idx / K4);
    const int k = (int)(idx % K4) * 4;
    uint32_t out = 0;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const float4 v = *reinterpret_cast<const float4 *>(W + (int64_t)(i * R + r) * K + k);
        out |= (uint32_t)!(v.x < 0.0f) << i;
        out |= (uint32_t)!(v.y < 0.0f) << (8 + i);
        out |= (uint32_t)!(v.z < 0.0f) << (16 + i);
        out |= (uint32_t)!(v.w < 0.0f) << (24 + i);
    }
    *reinterpret_cast<uint32_t *>(P + (int64_t)r * K + k) = out;
}

// ---------------------------------------------------------------------------
// Layer normalization + absmax int8, one workgroup per row.  Thread t holds
// the float4 chunks t + 256 j.  Sums in fixed order: per thread, the wave's
// butterfly, then the four waves pairwise.
// ---------------------------------------------------------------------------
__device__ __forceinline__ double block_sum(double v, double *red) {
    v = wave_sum(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const double r = (red[0] + red[1]) + (red[2] + red[3]);
    __syncthreads();
    return r;
}

__device__ __forceinline__ float block_max(float v, float *red) {
    v = wave_max(v);
    if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
    __syncthreads();
    const float r = fmaxf(fmaxf(red[0], red[1]), fmaxf(red[2], red[3]));
    __syncthreads();
    return r;
}

// NCH: float4 chunks per thread, the smallest count that covers the
// launch's largest K (the unrolled loops do no work past it).
template <int NCH>
__global__ __launch_bounds__(kT) void k_ln_quant(W1Batch unused) {
    (void)unused;
    __shared__ double red_d[4];
    __shared__ float red_f[4];
    const W1Batch &b = batch();
    int m = 0;
    const int p = problem_of(b, m);
    const W1Problem &pr = b.p[p];
    const int K = pr.K, nc = K >> 2, t = threadIdx.x;
    float v[NCH][4];
    if (pr.x_dt == BL_BF16) {
        const uint16_t *row = static_cast<const uint16_t *>(pr.x) + (size_t)m * pr.ldx;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = t + kT * j;
            uint2 u = make_uint2(0u, 0u);
            if (c < nc) u = *reinterpret_cast<const uint2 *>(row + 4 * c);
            v[j][0] = __uint_as_float(u.x << 16); v[j][1] = __uint_as_float(u.x & 0xFFFF0000u);
            v[j][2] = __uint_as_float(u.y << 16); v[j][3] = __uint_as_float(u.y & 0xFFFF0000u);
        }
    } else {
        const float *row = static_cast<const float *>(pr.x) + (size_t)m * pr.ldx;
#pragma unroll
        for (int j = 0; j < NCH; ++j) {
            const int c = t + kT * j;
            float4 u = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (c < nc) u = *reinterpret_cast<const float4 *>(row + 4 * c);
            v[j][0] = u.x; v[j][1] = u.y; v[j][2] = u.z; v[j][3] = u.w;
        }
    }
    double s = 0.0;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
#pragma unroll
        for (int f = 0; f < 4; ++f) s += (double)v[j][f];   // chunks past K hold zeros
    const double mu = block_sum(s, red_d) / (double)K;
    double ss = 0.0;
#pragma unroll
    for (int j = 0; j < NCH; ++j)
        if (t + kT * j < nc)
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const double d = (double)v[j][f] - mu;
                ss += d * d;
                v[j][f] = (float)d;   // the normalization needs only float(x - mu)
            }
    const double var = block_sum(ss, red_d) / (double)K;
    const float r = (float)(1.0 / sqrt(var + (double)b.eps));
    float am = 0.0f;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c = t + kT * j;
        if (c < nc) {
            float4 g = make_float4(1.0f, 1.0f, 1.0f, 1.0f), be = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
            if (pr.gamma) g = *reinterpret_cast<const float4 *>(pr.gamma + 4 * c);
            if (pr.beta) be = *reinterpret_cast<const float4 *>(pr.beta + 4 * c);
            const float gg[4] = {g.x, g.y, g.z, g.w}, bb[4] = {be.x, be.y, be.z, be.w};
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                float o = v[j][f] * r;   // float(x - mu) * r
                if (pr.gamma) o = o * gg[f];
                if (pr.beta) o = o + bb[f];
                v[j][f] = o;
                am = fmaxf(am, fabsf(o));
            }
        }
    }
    const float a = 127.0f / fmaxf(block_max(am, red_f), 1e-5f);
    int8_t *qrow = pr.q + (size_t)m * K;
#pragma unroll
    for (int j = 0; j < NCH; ++j) {
        const int c = t + kT * j;
        if (c < nc) {
            uint32_t w = 0;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int qi = (int)__builtin_amdgcn_fmed3f(rintf(v[j][f] * a), -128.0f, 127.0f);
                w |= ((uint32_t)qi & 0xFFu) << (8 * f);
            }
            *reinterpret_cast<uint32_t *>(qrow + 4 * c) = w;
        }
    }
    if (t == 0) pr.a[m] = a;
}

// ---------------------------------------------------------------------------
// Contraction.  Workgroup tile: 16 packed rows (128 output columns, 8 bit
// planes) x 16 NT tokens; the four waves split K step by step (wave w takes
// the 64-k steps w, w + 4, ...), issuing U steps' loads before consuming
// them, and meet through LDS integer adds at the end.  Loads read clamped,
// always valid addresses; operands outside M, R or K are zeroed in the
// consume phase.
// ---------------------------------------------------------------------------
__device__ __forceinline__ void planes(v4i b, v4i f[8]) {
#pragma unroll
    for (int i = 0; i < 7; ++i) f[i] = b & (0x01010101 << i);
    f[7] = (b >> 1) & 0x40404040;
}

template <int NT, int U>
__global__ __launch_bounds__(kT) void k_w1_gemm(W1Batch unused) {
    (void)unused;
    __shared__ int red[NT][8][64][4];
    __shared__ int qsm[NT * 16];
    const W1Batch &b = batch();
    int local = 0;
    const int p = problem_of(b, local);
    const W1Problem &pr = b.p[p];
    const int K = pr.K, M = pr.M, R = pr.N >> 3;
    const int nrg = (R + 15) >> 4;
    const int r0 = (local % nrg) * 16, m0 = (local / nrg) * 16 * NT;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;

    for (int i = tid; i < NT * 8 * 64 * 4; i += kT) (&red[0][0][0][0])[i] = 0;
    if (tid < NT * 16) qsm[tid] = 0;

    const bool row_ok = r0 + lr < R;
    const uint8_t *pb = pr.P + (size_t)(row_ok ? r0 + lr : 0) * K;
    const int8_t *pa[NT];
    bool tok_ok[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) {
        const int m = m0 + 16 * t + lr;
        tok_ok[t] = m < M;
        pa[t] = pr.q + (size_t)(tok_ok[t] ? m : 0) * K;
    }
    const int nst = (K + 63) >> 6;
    v4i acc[NT][8];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[t][i] = v4i{0, 0, 0, 0};
    int qs[NT];
#pragma unroll
    for (int t = 0; t < NT; ++t) qs[t] = 0;

    for (int s0 = wave; s0 < nst; s0 += 4 * U) {
        v4i bw[U], av[U][NT];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = s0 + 4 * u;
            int kk = (st < nst ? st : nst - 1) * 64 + 16 * g;
            kk = kk < K ? kk : K - 16;
            bw[u] = ld16(pb + kk);
#pragma unroll
            for (int t = 0; t < NT; ++t) av[u][t] = ld16(pa[t] + kk);
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int st = s0 + 4 * u;
            const bool k_ok = st < nst && st * 64 + 16 * g < K;
            const v4i z = v4i{0, 0, 0, 0};
            v4i f[8];
            planes((k_ok && row_ok) ? bw[u] : z, f);
#pragma unroll
            for (int t = 0; t < NT; ++t) {
                const v4i a = (k_ok && tok_ok[t]) ? av[u][t] : z;
                qs[t] += rowsum16(a);
#pragma unroll
                for (int i = 0; i < 8; ++i) acc[t][i] = mfma16(a, f[i], acc[t][i]);
            }
        }
    }
    __syncthreads();   // LDS cleared
#pragma unroll
    for (int t = 0; t < NT; ++t) {
#pragma unroll
        for (int i = 0; i < 8; ++i)
#pragma unroll
            for (int j = 0; j < 4; ++j) atomicAdd(&red[t][i][lane][j], acc[t][i][j]);
        int s = qs[t];
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        if (g == 0) atomicAdd(&qsm[16 * t + lr], s);
    }
    __syncthreads();
    // epilogue: wave w writes bit planes 2w and 2w + 1
    if (!row_ok) return;
    const float wsc = pr.w_scale[0];
#pragma unroll
    for (int t = 0; t < NT; ++t)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const int tl = 16 * t + 4 * g + j;
            const int m = m0 + tl;
            if (m >= M) continue;
            const float sc = wsc / pr.a[m];
            const int qsum = qsm[tl];
#pragma unroll
            for (int h = 0; h < 2; ++h) {
                const int i = 2 * wave + h;
                const int d = red[t][i][lane][j] >> (i < 7 ? i : 6);
                const int A = 2 * d - qsum;
                pr.y[(size_t)m * pr.N + (size_t)i * R + r0 + lr] = (float)A * sc;
            }
        }
}

// ---------------------------------------------------------------------------
// Contraction, large tiles (K a multiple of 128): 128 tokens x 32 packed rows
// (256 output columns over the 8 bit planes) per 4-wave workgroup, waves in
// a 2 x 2 grid (64 tokens x 16 packed rows each), two workgroups per CU.
// K advances in stages of 128 bytes per row through a 3-stage LDS ring fed
// by direct global->LDS loads (1 KB = 8 whole rows per load); one workgroup
// barrier per stage publishes stage s and certifies that every wave is done
// with stage s - 1, whose slot the loads of stage s + 2 reuse.  The 16-byte
// chunk c of tile row r sits at c ^ ((r >> 1) & 7), so a fragment read (16
// rows, one chunk each) spreads over all banks.  Each packed fragment is
// split into its 8 bit planes in registers and goes through the matrix cores
// once per plane with the weights as the first operand: lane (g, l) ends
// with packed rows 4 g .. 4 g + 3 of token l, four consecutive output
// columns of plane p (column p * N/8 + packed row).  The tokens' code sums
// come from the same operand reads.  Rows past M or N/8 read row 0 and are
// never stored.
// ---------------------------------------------------------------------------
constexpr int kWBK = 128;                        // k bytes per stage
constexpr int kWBStages = 3;
constexpr int kWBTM = 128;                       // tokens per tile
constexpr int kWBTR = 32;                        // packed rows per tile
constexpr int kWBA = kWBTM * kWBK;               // A bytes per stage
constexpr int kWBStage = kWBA + kWBTR * kWBK;    // 20 KB
constexpr int kWBDA = kWBA / (4 * 1024);         // 1 KB loads of A per wave per stage
constexpr int kWBDB = kWBTR * kWBK / (4 * 1024); // of B
constexpr int kWBDW = kWBDA + kWBDB;

template <int VM>
__device__ __forceinline__ void wb_wait_vm() {
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | (0x7 << 4) | (0xF << 8) | ((VM >> 4) << 14));
}

__device__ __forceinline__ void wb_dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

// Tiles of problem p: ceil(M / 128) token tiles x ceil(N/8 / 32) row tiles.
__host__ __device__ inline int wb_tiles(int M, int N) {
    return ((M + kWBTM - 1) / kWBTM) * ((N / 8 + kWBTR - 1) / kWBTR);
}

template <bool VOUT>
__global__ __launch_bounds__(kT) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_w1_gemm_big(W1Batch unused) {
    (void)unused;
    __shared__ __attribute__((aligned(16))) unsigned char lds[kWBStages * kWBStage];
    const W1Batch &b = batch();
    int local = 0;
    const int p = problem_of(b, local);
    const W1Problem &pr = b.p[p];
    const int K = pr.K, M = pr.M, N = pr.N, R = N >> 3;
    const int ntm = (M + kWBTM - 1) / kWBTM;
    const int m0 = (local % ntm) * kWBTM, r0 = (local / ntm) * kWBTR;
    const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63, lr = lane & 15, g = lane >> 4;
    const int wm = wave & 1, wn = wave >> 1;
    const int nst = K / kWBK;
    auto swz = [](int r) { return (r >> 1) & 7; };

    // this lane's part of each 1 KB load: row lane / 8 of the load's 8, chunk slot lane % 8
    const int lrow = lane >> 3, lpos = lane & 7;
    const int8_t *a_src[kWBDA];
#pragma unroll
    for (int i = 0; i < kWBDA; ++i) {
        const int row = (wave * kWBDA + i) * 8 + lrow;
        const int m = m0 + row < M ? m0 + row : 0;
        a_src[i] = pr.q + (size_t)m * K + 16 * (lpos ^ swz(row));
    }
    const uint8_t *b_src[kWBDB];
#pragma unroll
    for (int i = 0; i < kWBDB; ++i) {
        const int row = (wave * kWBDB + i) * 8 + lrow;
        const int r = r0 + row < R ? r0 + row : 0;
        b_src[i] = pr.P + (size_t)r * K + 16 * (lpos ^ swz(row));
    }
    auto issue = [&](int st) {
        unsigned char *base = lds + (st % kWBStages) * kWBStage;
        const size_t k0 = (size_t)st * kWBK;
#pragma unroll
        for (int i = 0; i < kWBDA; ++i) wb_dma16(a_src[i] + k0, base + (wave * kWBDA + i) * 1024);
#pragma unroll
        for (int i = 0; i < kWBDB; ++i) wb_dma16(b_src[i] + k0, base + kWBA + (wave * kWBDB + i) * 1024);
    };

    v4i acc[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int q = 0; q < 8; ++q) acc[i][q] = v4i{0, 0, 0, 0};
    int qs[4] = {0, 0, 0, 0};
    int aoff[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) aoff[i] = (wm * 64 + i * 16 + lr) * kWBK;
    const int boff = kWBA + (wn * 16 + lr) * kWBK;
    const int lsw = swz(lr);   // fragment rows start at multiples of 16
    auto chunk = [&](int ch) { return 16 * (ch ^ lsw); };

    lds_barrier();
    issue(0);
    if (nst > 1) issue(1);
    for (int st = 0; st < nst; ++st) {
        if (st + 1 < nst) wb_wait_vm<kWBDW>();
        else wb_wait_vm<0>();
        lds_barrier();
        const unsigned char *base = lds + (st % kWBStages) * kWBStage;
        v4i af[4], bw;
#pragma unroll
        for (int i = 0; i < 4; ++i) af[i] = *reinterpret_cast<const v4i *>(base + aoff[i] + chunk(g));
        bw = *reinterpret_cast<const v4i *>(base + boff + chunk(g));
#pragma unroll
        for (int ks = 0; ks < kWBK / 64; ++ks) {
            v4i an[4], bn;
            if (ks + 1 < kWBK / 64) {
                const int ch = 4 * (ks + 1) + g;
#pragma unroll
                for (int i = 0; i < 4; ++i) an[i] = *reinterpret_cast<const v4i *>(base + aoff[i] + chunk(ch));
                bn = *reinterpret_cast<const v4i *>(base + boff + chunk(ch));
            }
            v4i f[8];
            planes(bw, f);
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                qs[i] += rowsum16(af[i]);
#pragma unroll
                for (int q = 0; q < 8; ++q) acc[i][q] = mfma16(f[q], af[i], acc[i][q]);
            }
            // stage st + 2's loads after the first k-step's products (its
            // slot was freed at this stage's barrier)
            if (ks == 0 && st + 2 < nst) issue(st + 2);
            if (ks + 1 < kWBK / 64) {
#pragma unroll
                for (int i = 0; i < 4; ++i) af[i] = an[i];
                bw = bn;
            }
        }
    }

    // Epilogue: A = 2 (S >> plane shift) - (token code sum); y = float(A) * (w_scale / a).
    const float wsc = pr.w_scale[0];
    const int vr0 = r0 + wn * 16 + 4 * g;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        int s = qs[i];
        s += __shfl_xor(s, 16, 64);
        s += __shfl_xor(s, 32, 64);
        const int m = m0 + wm * 64 + i * 16 + lr;
        if (m >= M || vr0 >= R) continue;
        const float sc = wsc / pr.a[m];
        float *yrow = pr.y + (size_t)m * N;
#pragma unroll
        for (int q = 0; q < 8; ++q) {
            const int sh = q < 7 ? q : 6;
            float v[4];
#pragma unroll
            for (int j = 0; j < 4; ++j) v[j] = (float)(2 * (acc[i][q][j] >> sh) - s) * sc;
            if (VOUT) {
                *reinterpret_cast<float4 *>(yrow + (size_t)q * R + vr0) = make_float4(v[0], v[1], v[2], v[3]);
            } else {
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    if (vr0 + j < R) yrow[(size_t)q * R + vr0 + j] = v[j];
            }
        }
    }
}

// ---------------------------------------------------------------------------
// Decode (M = 1, K a multiple of 256 up to 8192): norm, quantization and
// contraction in one launch.  One 16-wave workgroup per 16 packed rows over
// all of K, cut into units of 4 packed rows x 256 bytes (lane (g, l) loads
// row l / 4, 16-byte chunk l % 4 + 4 g: every row arrives as two whole
// 128-byte lines).  Two roles:
//   * 8 quantizer waves load the input row (and gains), normalize and
//     quantize it into LDS; they issue no weight load, and they meet each
//     other through LDS flags, not workgroup barriers;
//   * 8 stream waves issue all their units at once (two waves per row quad,
//     alternate k-units; a fixed count, past-the-end units reading a valid
//     address), once every quantizer wave has issued its loads (requests
//     leave a compute unit in issue order: row loads issued behind the weight
//     stream would arrive after it), and then wait for the codes.  A wave that issues many loads stalls in the
//     issue itself while the compute unit drains them, so a barrier shared
//     with the quantization would wait for the stream.
// A unit goes through the matrix cores once per bit plane, weights first:
// product row 4 r + s is (unit row r, k-slice s), and column j of the codes
// operand carries k-slice j % 4 of the same chunks, so entry (4 r + s, s) is
// row r's sum over slice s; the four slices of a row sit in one lane quad
// and are added there, once per wave after all its units (the products of a
// wave's units accumulate in the matrix cores).  The row sums meet in LDS
// (integer adds).
// ---------------------------------------------------------------------------
constexpr int kDQW = 8;                      // quantizer waves (sum8 / max8 read eight partials)
constexpr int kDSW = 8;                      // stream waves
constexpr int kDT = (kDQW + kDSW) * 64;
constexpr int kDQT = kDQW * 64;
constexpr int kDU = 16;                      // k-units per stream wave: at least two waves per row quad, K / 256 <= 32
constexpr int kDUnitsCap = 5;                // k-units per stream wave above which tiles shrink
constexpr int kDChunks = 8192 / 4 / kDQT;         // float4 input chunks per quantizer thread

// Workgroup barrier waiting for LDS operations only; the scheduling fences
// keep the compiler from moving arithmetic (and the waits for its loaded
// operands) across it.
__device__ __forceinline__ void d_barrier() {
    __builtin_amdgcn_sched_barrier(0);
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    asm volatile("s_barrier" ::: "memory");
    __builtin_amdgcn_sched_barrier(0);
}

// The eight per-wave partials of an exchange, read as 16-byte vectors:
// their sum in wave order, their maximum.
__device__ __forceinline__ double sum8(const double *p) {
    const double2 a = reinterpret_cast<const double2 *>(p)[0], b = reinterpret_cast<const double2 *>(p)[1];
    const double2 c = reinterpret_cast<const double2 *>(p)[2], d = reinterpret_cast<const double2 *>(p)[3];
    return ((((((a.x + a.y) + b.x) + b.y) + c.x) + c.y) + d.x) + d.y;
}

__device__ __forceinline__ float max8(const float *p) {
    const float4 a = reinterpret_cast<const float4 *>(p)[0], b = reinterpret_cast<const float4 *>(p)[1];
    return fmaxf(fmaxf(fmaxf(a.x, a.y), fmaxf(a.z, a.w)), fmaxf(fmaxf(b.x, b.y), fmaxf(b.z, b.w)));
}

// The quantizer waves' rendezvous: each publishes `step` in its LDS flag and
// waits until every flag reaches it (bounded; an expired wait is counted and
// the wave goes on).
__device__ unsigned int g_w1_expired = 0;

// A poll is two 16-byte LDS reads (one wait) and scalar compares: read one
// flag at a time, each behind its own wait, a poll took about 0.4 us and a
// rendezvous up to two of them.  The compiler memory clobbers make every poll
// read LDS again and keep the flag store and the partials' reads in place.
__device__ __forceinline__ void q_sync(int *flag, int qw, int step) {
    static_assert(kDQW == 8, "two 16-byte reads cover the flags");
    __builtin_amdgcn_s_waitcnt(0xC07F);   // this wave's partials are in LDS
    asm volatile("" ::: "memory");
    if ((threadIdx.x & 63) == 0) flag[qw] = step;
    int lo = 0;
    for (int it = 0; it < (1 << 22); ++it) {
        asm volatile("" ::: "memory");
        const v4i f = *reinterpret_cast<const v4i *>(flag);
        const v4i h = *reinterpret_cast<const v4i *>(flag + 4);
        lo = step;
#pragma unroll
        for (int i = 0; i < 4; ++i)
            lo = min(lo, min(__builtin_amdgcn_readfirstlane(f[i]), __builtin_amdgcn_readfirstlane(h[i])));
        if (lo >= step) break;
    }
    if (lo < step && (threadIdx.x & 63) == 0) atomicAdd(&g_w1_expired, 1u);
    asm volatile("" ::: "memory");
}

template <bool BF16>
__global__ __launch_bounds__(kDT) void k_w1_decode(W1Batch unused) {
    (void)unused;
    __shared__ __attribute__((aligned(16))) int8_t qd[8192];
    __shared__ int red[8][16];
    __shared__ __attribute__((aligned(16))) double rd1[kDQW];   // per-wave sums of x
    __shared__ __attribute__((aligned(16))) double rd2[kDQW];   // per-wave sums of (x - mu)^2
    __shared__ __attribute__((aligned(16))) float rm[kDQW];     // per-wave max |float(x - mu)|
    __shared__ __attribute__((aligned(16))) float rf[kDQW];     // per-wave max |x'| (with gain or bias)
    __shared__ int ri[kDQW];
    __shared__ __attribute__((aligned(16))) int flag[kDQW];
    const W1Batch &b = batch();
    int local = 0, quads = 1;
    const int p = problem_of(b, local, &quads);
    const W1Problem &pr = b.p[p];
    const int K = pr.K, R = pr.N >> 3, nku = K >> 8, nu = 4 * nku;
    // every field of the problem read here together (the compiler would
    // issue each load next to its first use, one round trip after another)
    asm volatile("" ::"s"(K), "s"(R), "s"(pr.x), "s"(pr.gamma), "s"(pr.beta), "s"(pr.w_scale), "s"(pr.P), "s"(pr.y));
    const int tid = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(tid >> 6), lane = tid & 63, g = lane >> 4;
    const int lq = quads == 4 ? 2 : (quads == 2 ? 1 : 0);   // log2 of the row quads
    const int r0 = local * (4 << lq);
    float a = 1.0f;

    if (wave < kDQW) {
        // ---- quantizer waves: the row, its norm and its codes
        const int nc = K >> 2;
        if (lane == 0) flag[wave] = 0;
        if (tid < 8 * 16) (&red[0][0])[tid] = 0;
        // every load unconditional, at a clamped valid address (chunks past K
        // read chunk 0; absent gains read 16 bytes of the row itself, at an
        // offset of their own per lane: one address shared by every lane of
        // the launch would queue on one L2 channel), zeroed or replaced
        // afterwards: a branch around a load would make the compiler wait for
        // the loads before it
        float xv[kDChunks][4];
        uint2 xb[kDChunks];
        float4 xf[kDChunks], gq[kDChunks], bq[kDChunks];
        const float *xrow = static_cast<const float *>(pr.x);
        const int xfl = BF16 ? K / 2 : K;   // the row's length in floats
#pragma unroll
        for (int i = 0; i < kDChunks; ++i) {
            const int c = tid + kDQT * i;
            const int cc = c < nc ? c : 0;
            if (BF16) xb[i] = *reinterpret_cast<const uint2 *>(static_cast<const uint16_t *>(pr.x) + 4 * cc);
            else xf[i] = *reinterpret_cast<const float4 *>(static_cast<const float *>(pr.x) + 4 * cc);
            const int xo = 4 * cc < xfl ? 4 * cc : 4 * cc - xfl;   // < xfl - 3: in the row
            gq[i] = *reinterpret_cast<const float4 *>(pr.gamma ? pr.gamma + 4 * cc : xrow + xo);
            bq[i] = *reinterpret_cast<const float4 *>(pr.beta ? pr.beta + 4 * cc : xrow + xo);
        }
        // the weight scale for the epilogue, fetched with the row (read at
        // the end it would be a memory round trip behind the weight stream)
        const float wsc = pr.w_scale[0];
        d_barrier();   // every row and gain load issued: the weight stream may start
#pragma unroll
        for (int i = 0; i < kDChunks; ++i) {
            const bool ok = tid + kDQT * i < nc;
            if (BF16) {
                const uint2 u = ok ? xb[i] : make_uint2(0u, 0u);
                xv[i][0] = __uint_as_float(u.x << 16); xv[i][1] = __uint_as_float(u.x & 0xFFFF0000u);
                xv[i][2] = __uint_as_float(u.y << 16); xv[i][3] = __uint_as_float(u.y & 0xFFFF0000u);
            } else {
                const float4 u = ok ? xf[i] : make_float4(0.0f, 0.0f, 0.0f, 0.0f);
                xv[i][0] = u.x; xv[i][1] = u.y; xv[i][2] = u.z; xv[i][3] = u.w;
            }
            if (!pr.gamma) gq[i] = make_float4(1.0f, 1.0f, 1.0f, 1.0f);
            if (!pr.beta) bq[i] = make_float4(0.0f, 0.0f, 0.0f, 0.0f);
        }
        double s = 0.0;
#pragma unroll
        for (int i = 0; i < kDChunks; ++i)
#pragma unroll
            for (int f = 0; f < 4; ++f) s += (double)xv[i][f];   // chunks past K hold zeros
        s = wave_sum_dpp(s);
        if (lane == 0) rd1[wave] = s;
        q_sync(flag, wave, 1);
        // each exchange has its own slots, so no wave waits for the others'
        // reads before writing the next one; the partials are read as
        // 16-byte vectors and added in wave order
        const double mu = sum8(rd1) / (double)K;
        double ss = 0.0;
        float md = 0.0f;
#pragma unroll
        for (int i = 0; i < kDChunks; ++i)
            if (tid + kDQT * i < nc)
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const double d = (double)xv[i][f] - mu;
                    ss += d * d;
                    xv[i][f] = (float)d;   // the normalization below needs only float(x - mu)
                    md = fmaxf(md, fabsf(xv[i][f]));
                }
        ss = wave_sum_dpp(ss);
        md = wave_max_dpp(md);
        if (lane == 0) {
            rd2[wave] = ss;
            rm[wave] = md;
        }
        q_sync(flag, wave, 2);
        const float r = (float)(1.0 / sqrt(sum8(rd2) / (double)K + (double)b.eps));
        const bool affine = pr.gamma || pr.beta;
        float mx = 0.0f;
        if (!affine) {
            // without gain or bias the largest |float(x - mu) * r| is
            // float(max |float(x - mu)| * r): the rounded product is monotone
            // in the first factor and odd, so the maximum commutes with it
            mx = max8(rm) * r;
        }
#pragma unroll
        for (int i = 0; i < kDChunks; ++i) {
            const int c = tid + kDQT * i;
            const float gg[4] = {gq[i].x, gq[i].y, gq[i].z, gq[i].w}, bb[4] = {bq[i].x, bq[i].y, bq[i].z, bq[i].w};
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                float o = xv[i][f] * r;   // float(x - mu) * r
                if (pr.gamma) o = o * gg[f];
                if (pr.beta) o = o + bb[f];
                xv[i][f] = c < nc ? o : 0.0f;
            }
        }
        if (affine) {
            float am = 0.0f;
#pragma unroll
            for (int i = 0; i < kDChunks; ++i)
#pragma unroll
                for (int f = 0; f < 4; ++f) am = fmaxf(am, fabsf(xv[i][f]));
            am = wave_max_dpp(am);
            if (lane == 0) rf[wave] = am;
            q_sync(flag, wave, 3);
            mx = max8(rf);
        }
        a = 127.0f / fmaxf(mx, 1e-5f);
        int cs = 0;
#pragma unroll
        for (int i = 0; i < kDChunks; ++i) {
            const int c = tid + kDQT * i;
            if (c < nc) {
                uint32_t w = 0;
#pragma unroll
                for (int f = 0; f < 4; ++f) {
                    const int qi = (int)__builtin_amdgcn_fmed3f(rintf(xv[i][f] * a), -128.0f, 127.0f);
                    w |= ((uint32_t)qi & 0xFFu) << (8 * f);
                    cs += qi;
                }
                *reinterpret_cast<uint32_t *>(qd + 4 * c) = w;
            }
        }
        cs = wave_sum_dpp(cs);
        if (lane == 0) ri[wave] = cs;
        d_barrier();   // codes in LDS
        // while the stream waves multiply: the code sum and w_scale / a (IEEE
        // fp32 division), so that only the row sum's read, a subtraction, a
        // conversion, a multiply and the store follow the last barrier
        int qsum = 0;
#pragma unroll
        for (int w = 0; w < kDQW; ++w) qsum += ri[w];
        const float sc = wsc / a;
        d_barrier();   // row sums in LDS
        if (lane < (4 << lq) && r0 + lane < R) {   // wave w writes bit plane w
            const int i = wave;
            const int A = 2 * (red[i][lane] >> (i < 7 ? i : 6)) - qsum;
            pr.y[(size_t)i * R + r0 + lane] = (float)A * sc;
        }
    } else {
        // ---- stream waves: every unit issued, then the products.  With Q
        // row quads, wave w takes quad w % Q and every (8 / Q)-th 256-byte
        // k-unit from w / Q, so its products accumulate in the matrix cores'
        // accumulators
        const int sw = wave - kDQW, q = sw & ((1 << lq) - 1), k0 = sw >> lq, kst = kDSW >> lq;
        const int urow = (lane & 15) >> 2, ch = (lane & 3) + 4 * g;
        int row = r0 + 4 * q + urow;
        const bool row_ok = row < R;
        row = row_ok ? row : R - 1;
        const uint8_t *pw = pr.P + (size_t)row * K + 16 * ch;
        d_barrier();   // the quantizer waves' loads go out first
        v4i bw[kDU];
#pragma unroll
        for (int j = 0; j < kDU; ++j) {
            int ku = k0 + kst * j;
            ku = ku < nku ? ku : nku - 1;
            bw[j] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(pw + ku * 256));
        }
        d_barrier();   // codes in LDS
        v4i acc[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) acc[i] = v4i{0, 0, 0, 0};
#pragma unroll
        for (int j = 0; j < kDU; ++j) {
            const int ku = k0 + kst * j;
            if (ku >= nku) break;   // uniform; the loads above were issued for every j
            const v4i cw = *reinterpret_cast<const v4i *>(qd + ku * 256 + 16 * ch);
            v4i f[8];
            planes(row_ok ? bw[j] : v4i{0, 0, 0, 0}, f);
#pragma unroll
            for (int i = 0; i < 8; ++i) acc[i] = mfma16(f[i], cw, acc[i]);
        }
        const int sl = lane & 3;
        int t[8];
#pragma unroll
        for (int i = 0; i < 8; ++i)
            t[i] = quad_sum(sl == 0 ? acc[i][0] : (sl == 1 ? acc[i][1] : (sl == 2 ? acc[i][2] : acc[i][3])));
        if ((lane & 15) == 0)
#pragma unroll
            for (int i = 0; i < 8; ++i) atomicAdd(&red[i][4 * q + g], t[i]);
        d_barrier();   // row sums in LDS
    }
}

} // namespace

// Workspace and shape rules for the host side (bl_api.hip).
int w1_ln_max_k() { return kLnMaxChunks * kT * 4; }

hipError_t launch_binarize_pack(const float *W, int N, int K, uint8_t *packed, hipStream_t s) {
    const int64_t n = (int64_t)(N / 8) * (K / 4);
    hipLaunchKernelGGL(k_binarize_pack4, dim3((unsigned)((n + kT - 1) / kT)), dim3(kT), 0, s, W, N, K, packed);
    return hipGetLastError();
}

static W1Problem to_problem(const W1Args &a) {
    return W1Problem{a.x, a.x_dt, a.ldx, a.gamma, a.beta, a.M, a.K, a.q, a.a, a.P, a.N, a.w_scale, a.y};
}

// One launch of the norm over the rows of b, with NCH = nch.
static hipError_t launch_ln(int nch, const W1Batch &b, int rows, hipStream_t s) {
    switch (nch) {
#define BL_LN_CASE(c) \
    case c: hipLaunchKernelGGL(k_ln_quant<c>, dim3(rows), dim3(kT), 0, s, b); break;
        BL_LN_CASE(1) BL_LN_CASE(2) BL_LN_CASE(3) BL_LN_CASE(4) BL_LN_CASE(5) BL_LN_CASE(6) BL_LN_CASE(7) BL_LN_CASE(8)
        BL_LN_CASE(9) BL_LN_CASE(10) BL_LN_CASE(11) BL_LN_CASE(12) BL_LN_CASE(13) BL_LN_CASE(14) BL_LN_CASE(15)
        BL_LN_CASE(16)
#undef BL_LN_CASE
    default: return hipErrorInvalidValue;   // K above kLnMaxChunks * kT * 4 (host-checked)
    }
    return hipGetLastError();
}

// The norm and quantization of every row of the problems (x, gamma, beta in;
// q, a out), one launch.  (One launch per chunk count measured the same:
// the kernel is bound by each row's chain of loads and reductions, not by
// the unrolled arithmetic.)
hipError_t launch_w1_norm(const W1Args *probs, int n, float eps, hipStream_t s) {
    W1Batch b{};
    b.n = n;
    b.eps = eps;
    int rows = 0, maxk = 4;
    for (int i = 0; i < n; ++i) {
        b.p[i] = to_problem(probs[i]);
        b.start[i] = rows;
        rows += probs[i].M;
        maxk = probs[i].K > maxk ? probs[i].K : maxk;
    }
    b.start[n] = rows;
    return launch_ln((maxk / 4 + kT - 1) / kT, b, rows, s);
}

hipError_t w1_wait_expired(unsigned int *count, bool reset) {
    unsigned int v = 0;
    if (hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_w1_expired), sizeof(v)); e != hipSuccess) return e;
    if (reset && v) {
        const unsigned int zero = 0;
        if (hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_w1_expired), &zero, sizeof(zero)); e != hipSuccess) return e;
    }
    *count = v;
    return hipSuccess;
}

bool w1_decode_fits(const W1Args *probs, int n) {
    for (int i = 0; i < n; ++i)
        if (probs[i].M != 1 || probs[i].K % 256 != 0 || probs[i].K > 8192 || !probs[i].x ||
            probs[i].x_dt != probs[0].x_dt)
            return false;
    return true;
}

// Decode: every problem at M = 1 (one input type, K a multiple of 256 up to
// 8192) in one launch (norm, quantization and contraction; q and a are not
// written).
hipError_t launch_w1_decode(const W1Args *probs, int n, float eps, hipStream_t s) {
    W1Batch b{};
    b.n = n;
    b.eps = eps;
    // the problems with the longest tiles (largest K) first: the device
    // starts the lowest workgroup numbers first
    int order[kMaxProblems];
    for (int i = 0; i < n; ++i) order[i] = i;
    for (int i = 1; i < n; ++i)
        for (int j = i; j > 0 && probs[order[j]].K > probs[order[j - 1]].K; --j) std::swap(order[j], order[j - 1]);
    // Row quads per workgroup: 4 (16 packed rows) unless that gives a
    // stream wave more than kDUnitsCap k-units (8 stream waves share the
    // workgroup's quads x K/256 units): the longest rows get smaller tiles,
    // so that no compute unit's matrix cores hold up the launch.
    int start = 0;
    for (int i = 0; i < n; ++i) {
        const W1Args &a = probs[order[i]];
        b.p[i] = to_problem(a);
        b.start[i] = start;
        int qd = 4;
        while (qd > 1 && qd * (a.K / 256) > kDUnitsCap * kDSW) qd >>= 1;
        b.quads[i] = qd;
        start += (a.N / 8 + 4 * qd - 1) / (4 * qd);
    }
    b.start[n] = start;
    if (probs[0].x_dt == BL_BF16)
        hipLaunchKernelGGL(k_w1_decode<true>, dim3(start), dim3(kDT), 0, s, b);
    else
        hipLaunchKernelGGL(k_w1_decode<false>, dim3(start), dim3(kDT), 0, s, b);
    return hipGetLastError();
}

// The contraction of every problem (q, a, P, w_scale in; y out), one launch.
hipError_t launch_w1_gemm(const W1Args *probs, int n, hipStream_t s) {
    W1Batch b{};
    b.n = n;
    // Large tiles when every K is whole 128-byte stages, the operands are
    // 16-byte aligned and the launch holds at least one tile per CU.
    bool big = true, vout = true;
    int big_tiles = 0;
    for (int i = 0; i < n; ++i) {
        const W1Args &a = probs[i];
        big = big && a.K % kWBK == 0 && (uintptr_t)a.q % 16 == 0 && (uintptr_t)a.P % 16 == 0;
        vout = vout && a.N % 32 == 0 && (uintptr_t)a.y % 16 == 0;
        big_tiles += wb_tiles(a.M, a.N);
    }
    if (big && big_tiles >= device_cu_count()) {
        int start = 0;
        for (int i = 0; i < n; ++i) {
            b.p[i] = to_problem(probs[i]);
            b.start[i] = start;
            start += wb_tiles(probs[i].M, probs[i].N);
        }
        b.start[n] = start;
        if (vout)
            hipLaunchKernelGGL(k_w1_gemm_big<true>, dim3(start), dim3(kT), 0, s, b);
        else
            hipLaunchKernelGGL(k_w1_gemm_big<false>, dim3(start), dim3(kT), 0, s, b);
        return hipGetLastError();
    }
    int max_m = 0;
    for (int i = 0; i < n; ++i) max_m = probs[i].M > max_m ? probs[i].M : max_m;
    const int nt = max_m > 16 ? 2 : 1;
    int start = 0;
    for (int i = 0; i < n; ++i) {
        b.p[i] = to_problem(probs[i]);
        b.start[i] = start;
        const int R = probs[i].N / 8;
        start += ((R + 15) / 16) * ((probs[i].M + 16 * nt - 1) / (16 * nt));
    }
    b.start[n] = start;
    if (nt == 1)
        hipLaunchKernelGGL((k_w1_gemm<1, 8>), dim3(start), dim3(kT), 0, s, b);
    else
        hipLaunchKernelGGL((k_w1_gemm<2, 4>), dim3(start), dim3(kT), 0, s, b);
    return hipGetLastError();
}

} // namespace bl
