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
// Code sums: s[m] = sum_k q[m,k], one workgroup per row (K a multiple of 16).
// The contraction takes codes + 1 from the packed fields and subtracts this
// sum once per output.
// ===========================================================================
__global__ __launch_bounds__(256) void k_code_sums(const int8_t *q, int ldq, int M, int K, int *out) {
    __shared__ int part[4];
    const int m = blockIdx.x;
    const int8_t *row = q + (size_t)m * ldq;
    int acc = 0;
    for (int k = threadIdx.x * 16; k < K; k += 256 * 16) acc += rowsum16(ld16(row + k));
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) acc += __shfl_xor(acc, o, 64);
    if ((threadIdx.x & 63) == 0) part[threadIdx.x >> 6] = acc;
    __syncthreads();
    if (threadIdx.x == 0) out[m] = part[0] + part[1] + part[2] + part[3];
}

// ===========================================================================
// Prefill kernel, large tiles (K a multiple of kGK).
// Workgroup: 4 waves in a 2 x 2 grid over a TM-token x TR-packed-row tile
// (PAIR: TR/2 gate rows and the same TR/2 up rows).  Wave (wm, wn) owns TM/2
// tokens (NA = TM/32 MFMA token tiles) and NBW 16-row weight fragments; each
// packed fragment is unpacked in registers into its four fields, so one
// fragment feeds 4 * NA MFMAs (v_mfma_i32_16x16x64_i8) per 64-k step.
// K advances in stages of kGK bytes per row, brought into a 3-stage LDS ring
// with direct global->LDS loads (one 1 KB load = 1024 / kGK whole rows).  One
// workgroup barrier per stage: every wave waits for its own loads of stage s,
// the barrier then publishes stage s and also certifies that every wave is
// done with stage s-1, whose slot the loads of stage s+2 reuse.  In LDS the
// 16-byte chunks of each tile row are XOR-swizzled (swz below) so that a
// fragment read (16 rows, one chunk each) spreads over all bank groups.
// ===========================================================================
constexpr int kGK = 128;     // k bytes per stage
constexpr int kGStages = 3;

template <bool PAIR, int TM, int NBW>
struct GemmShape {
    static constexpr int NA = TM / 32;               // 16-token tiles per wave
    static constexpr int BR = 32 * NBW;              // packed rows staged per stage
    static constexpr int A_BYTES = TM * kGK;
    static constexpr int B_BYTES = BR * kGK;
    static constexpr int STAGE = A_BYTES + B_BYTES;
    static constexpr int DPA = TM * kGK / 4096;      // 1 KB loads of A per wave per stage
    static constexpr int DPB = BR * kGK / 4096;
    static constexpr int DPW = DPA + DPB;            // 1 KB loads per wave per stage
    static constexpr int ROWS = PAIR ? BR / 2 : BR;  // packed rows of the output tile
    static_assert(!PAIR || NBW == 2, "a gate|up tile holds one gate and one up fragment per wave");
    static_assert(kGStages * DPW < 64, "vmcnt holds at most 63 loads");
};

template <int VM>
__device__ __forceinline__ void g_wait_vm() {
    __builtin_amdgcn_s_waitcnt((VM & 0xF) | (0x7 << 4) | (0xF << 8) | ((VM >> 4) << 14));
}

// Direct global->LDS load of 16 bytes per lane (lane l lands at lds + 16 l).
// (Target builtins stay inside device functions: used directly in a kernel
// template's body they would keep the host side from emitting its stub.)
__device__ __forceinline__ void g_dma16(const void *src, void *lds) {
    __builtin_amdgcn_global_load_lds(src, lds, 16, 0, 0);
}

__device__ __forceinline__ void g_lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0) only
    asm volatile("s_barrier" ::: "memory");
}

// One output tile: TM tokens from m0 x the packed rows from r0 (ROWS of them).
template <bool PAIR, int TM, int NBW, bool VOUT>
__device__ __forceinline__ void gemm_tile(const Contract &c, const int m0, const int r0, unsigned char *g_lds) {
    using S = GemmShape<PAIR, TM, NBW>;
    constexpr int NA = S::NA;
    const int tid = threadIdx.x;
    const int wave = tid >> 6;
    const int lane = tid & 63;
    const int lr = lane & 15;
    const int g = lane >> 4;
    const int wm = wave & 1;
    const int wn = wave >> 1;
    const int K = c.K;
    const int nst = K / kGK;
    // Swizzle of a tile row: the 16-byte chunk c of row r sits at position
    // c ^ swz(r).  With 256-byte rows a row spans all 64 banks, so the 16 rows
    // of a fragment need 16 distinct positions (r & 15); with 128-byte rows
    // two rows share the banks, so rows r and r + 1 need the same positions
    // offset by half a row: ((r >> 1) & 7).
    auto swz = [](int r) { return kGK == 256 ? (r & 15) : ((r >> 1) & 7); };

    // this lane's part of every 1 KB load: row L / CPR of the 1024 / kGK, chunk slot L % CPR
    constexpr int CPR = kGK / 16;                             // 16-byte chunks per row
    constexpr int RPL = 1024 / kGK;                           // rows per 1 KB load
    const int lrow = lane / CPR;
    const int lpos = lane % CPR;
    const int8_t *a_src[S::DPA];
#pragma unroll
    for (int i = 0; i < S::DPA; ++i) {
        const int row = (wave * S::DPA + i) * RPL + lrow;    // tile row 0 .. TM-1
        const int ch = lpos ^ swz(row);
        const int m = m0 + row < c.M ? m0 + row : 0;         // rows past M compute garbage never stored
        a_src[i] = c.q + (size_t)m * c.ldq + 16 * ch;
    }
    const uint8_t *b_src[S::DPB];
#pragma unroll
    for (int i = 0; i < S::DPB; ++i) {
        const int row = (wave * S::DPB + i) * RPL + lrow;    // B stage row 0 .. BR-1
        const int ch = lpos ^ swz(row);
        const int trow = PAIR ? (row < S::BR / 2 ? row : row - S::BR / 2) : row;   // row within its tensor's tile
        const int prow = (PAIR && row >= S::BR / 2 ? c.R : 0) + r0 + trow;
        const bool ok = r0 + trow < c.R;
        b_src[i] = c.P + (size_t)(ok ? prow : 0) * K + 16 * ch;
    }
    auto issue = [&](int st) {
        unsigned char *base = g_lds + (st % kGStages) * S::STAGE;
        const size_t k0 = (size_t)st * kGK;
#pragma unroll
        for (int i = 0; i < S::DPA; ++i) g_dma16(a_src[i] + k0, base + (wave * S::DPA + i) * 1024);
#pragma unroll
        for (int i = 0; i < S::DPB; ++i) g_dma16(b_src[i] + k0, base + S::A_BYTES + (wave * S::DPB + i) * 1024);
    };

    // Operand order: the unpacked weight fragment is the MFMA's first operand
    // and the activations the second, so lane (g, lr) accumulates packed rows
    // 4g .. 4g + 3 of a fragment for token lr: four consecutive output columns
    // of one token row.  The accumulators start at -(code sum of the token) x
    // (field scale), which removes the +1 of every code, and the field scale
    // (1, 4, 16, 16) divides out exactly at the end.
    int mtok[NA];
    float am[NA];
    v4i acc[NA][NBW][4];
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        mtok[i] = m0 + wm * (TM / 2) + i * 16 + lr;
        const bool okm = mtok[i] < c.M;
        const int qs = okm ? c.qsum[mtok[i]] : 0;
        am[i] = okm ? c.a[mtok[i]] : 1.0f;
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int v = -qs * (f == 0 ? 1 : (f == 1 ? 4 : 16));
#pragma unroll
            for (int b = 0; b < NBW; ++b) acc[i][b][f] = v4i{v, v, v, v};
        }
    }
    // LDS byte offsets of this lane's fragment rows (chunk 0 excluded)
    int aoff[NA];
#pragma unroll
    for (int i = 0; i < NA; ++i) aoff[i] = (wm * (TM / 2) + i * 16 + lr) * kGK;
    int boff[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b)
        boff[b] = S::A_BYTES + (PAIR ? (b == 0 ? wn * 16 + lr : S::BR / 2 + wn * 16 + lr) : (wn * NBW + b) * 16 + lr) * kGK;
    // the swizzled position of chunk ch for this lane's rows: rows of a fragment
    // are 16 consecutive tile rows starting at a multiple of 16, so their
    // swizzle is swz(lr)
    const int lsw = swz(lr);
    auto chunk = [&](int ch) { return 16 * (ch ^ lsw); };

    g_lds_barrier();   // the kernel's static LDS initialised; no LDS load below can race it
    issue(0);
    if (nst > 1) issue(1);
    v4i af[NA], bw[NBW];
    for (int st = 0; st < nst; ++st) {
        // this wave's loads of stage st are done once at most those of stage
        // st + 1 are outstanding
        if (st + 1 < nst) g_wait_vm<S::DPW>();
        else g_wait_vm<0>();
        g_lds_barrier();
        const unsigned char *base = g_lds + (st % kGStages) * S::STAGE;
        // Raised wave priority from the stage's operand reads to its last
        // product: of the two workgroups sharing a CU, the one with operands in
        // LDS issues first, the other's wait and barrier overlap it (3 %).
        __builtin_amdgcn_s_setprio(1);
        // operands of k-step 0
#pragma unroll
        for (int i = 0; i < NA; ++i) af[i] = *reinterpret_cast<const v4i *>(base + aoff[i] + chunk(g));
#pragma unroll
        for (int b = 0; b < NBW; ++b) bw[b] = *reinterpret_cast<const v4i *>(base + boff[b] + chunk(g));
#pragma unroll
        for (int ks = 0; ks < kGK / 64; ++ks) {
            v4i an[NA], bn[NBW];
            if (ks + 1 < kGK / 64) {
                const int ch = 4 * (ks + 1) + g;
#pragma unroll
                for (int i = 0; i < NA; ++i) an[i] = *reinterpret_cast<const v4i *>(base + aoff[i] + chunk(ch));
#pragma unroll
                for (int b = 0; b < NBW; ++b) bn[b] = *reinterpret_cast<const v4i *>(base + boff[b] + chunk(ch));
            }
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                // the four fields, masked in place: codes + 1 times 1, 4, 16, 16
                v4i f0, f1, f2, f3;
#pragma unroll
                for (int d = 0; d < 4; ++d) {
                    const uint32_t w = (uint32_t)bw[b][d];
                    f0[d] = (int)(w & 0x03030303u);
                    f1[d] = (int)(w & 0x0C0C0C0Cu);
                    f2[d] = (int)(w & 0x30303030u);
                    f3[d] = (int)((w >> 2) & 0x30303030u);
                }
#pragma unroll
                for (int i = 0; i < NA; ++i) {
                    acc[i][b][0] = mfma16(f0, af[i], acc[i][b][0]);
                    acc[i][b][1] = mfma16(f1, af[i], acc[i][b][1]);
                    acc[i][b][2] = mfma16(f2, af[i], acc[i][b][2]);
                    acc[i][b][3] = mfma16(f3, af[i], acc[i][b][3]);
                }
            }
            // The loads of stage st + 2 go out after the first k-step's
            // products (their slot was freed at this stage's barrier): the
            // matrix cores start right after the barrier (1.8 %).
            if (ks == 0 && st + 2 < nst) issue(st + 2);
            if (ks + 1 < kGK / 64) {
#pragma unroll
                for (int i = 0; i < NA; ++i) af[i] = an[i];
#pragma unroll
                for (int b = 0; b < NBW; ++b) bw[b] = bn[b];
            }
        }
        __builtin_amdgcn_s_setprio(0);
    }

    // Epilogue.  Lane (g, lr) holds, per token fragment i, weight fragment b
    // and field f, packed rows vr0 .. vr0 + 3 (vr0 a multiple of 4) of token
    // mtok[i]; they sit in consecutive output columns when the segment sizes
    // are multiples of 4 (checked by the launcher for the vector path).  The
    // factor w_mean / a is formed once per (token, segment) with IEEE fp32
    // division, as the oracle does; each output then costs a shift, a
    // conversion and a multiply: float(A) * (w_mean / a).
    int colb[NBW][4];
    float wmb[NBW];
    int vrb[NBW];
#pragma unroll
    for (int b = 0; b < NBW; ++b) {
        const int vr0 = r0 + (PAIR ? wn * 16 : (wn * NBW + b) * 16) + 4 * g;
        vrb[b] = vr0;
        const int vrc = vr0 < c.R ? vr0 : 0;
        if (PAIR) {
            // gate (b = 0) and up (b = 1) share the row; p goes to column f*R + vr
#pragma unroll
            for (int f = 0; f < 4; ++f) colb[b][f] = f * c.R + vrc;
            wmb[b] = c.w_mean[b];
        } else {
            int sg = 0;
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const ColOf co = col_of(c.seg, vrc, f);
                colb[b][f] = co.col;
                sg = co.seg;
            }
            wmb[b] = c.w_mean[sg];
        }
    }
#pragma unroll
    for (int i = 0; i < NA; ++i) {
        const int m = mtok[i];
        if (m >= c.M) continue;
        const size_t rowo = (size_t)m * c.ldy;
        if (PAIR) {
            if (vrb[0] >= c.R) continue;
            const float s0 = wmb[0] / am[i];
            const float s1 = wmb[1] / am[i];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int sh = f == 0 ? 0 : (f == 1 ? 2 : 4);
                float v[4];
#pragma unroll
                for (int j = 0; j < 4; ++j)
                    v[j] = relu2_mul((float)(acc[i][0][f][j] >> sh) * s0, (float)(acc[i][1][f][j] >> sh) * s1);
                if (VOUT) {
                    store4(c.y, c.y_dt, rowo + colb[0][f], v);
                } else {
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        if (vrb[0] + j >= c.R) break;
                        const size_t idx = rowo + colb[0][f] + j;
                        if (c.y_dt == BL_BF16) ((uint16_t *)c.y)[idx] = f32_to_bf16(v[j]);
                        else ((float *)c.y)[idx] = v[j];
                    }
                }
            }
        } else {
#pragma unroll
            for (int b = 0; b < NBW; ++b) {
                if (vrb[b] >= c.R) continue;
                if (VOUT) {
                    const float sc = wmb[b] / am[i];
#pragma unroll
                    for (int f = 0; f < 4; ++f) {
                        const int sh = f == 0 ? 0 : (f == 1 ? 2 : 4);
                        float v[4];
#pragma unroll
                        for (int j = 0; j < 4; ++j) {
                            const int A = acc[i][b][f][j] >> sh;
                            v[j] = c.y_dt == BL_I32 ? __int_as_float(A) : (float)A * sc;
                        }
                        store4(c.y, c.y_dt, rowo + colb[b][f], v);
                    }
                } else {
                    // scalar stores; the four rows may straddle a segment boundary
#pragma unroll
                    for (int j = 0; j < 4; ++j) {
                        const int vr = vrb[b] + j;
                        if (vr >= c.R) break;
#pragma unroll
                        for (int f = 0; f < 4; ++f) {
                            const int sh = f == 0 ? 0 : (f == 1 ? 2 : 4);
                            const ColOf co = col_of(c.seg, vr, f);
                            store_out(c.y, c.y_dt, rowo + co.col, acc[i][b][f][j] >> sh, c.w_mean[co.seg] / am[i]);
                        }
                    }
                }
            }
        }
    }
}

// Workgroup b of the launch: the leading nA workgroups take full tiles 0 ..
// nA - 1; the next nH take half tiles (TM / 2 tokens) covering full tiles nA
// .. nA + nH / 2 - 1; the rest take the remaining full tiles in order.  The
// device starts workgroups b and b + (number of CUs) on the same CU, so with
// nA = nH = CUs each CU's second workgroup finishes its first tile about half
// way through the first one's, and from then on the two run half a tile out
// of phase: one's epilogue (bound by the chip-wide output writes) overlaps
// the other's MFMA loop.  Tile t covers tokens (t % ntm) * TM and packed rows
// (t / ntm) * ROWS.
template <bool PAIR, int TM, int NBW, bool VOUT>
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2)))
void k_gemm_big(Contract c, int ntm, int nA, int nH) {
    using S = GemmShape<PAIR, TM, NBW>;
    // a static LDS object first: the dynamic ring must not start at address 0
    __shared__ int qs_s[4];
    extern __shared__ __attribute__((aligned(16))) unsigned char g_lds[];
    if (threadIdx.x < 4) qs_s[threadIdx.x] = 0;
    const int b = blockIdx.x;
    if constexpr (TM % 64 == 0) {
        if (b >= nA && b < nA + nH) {
            const int h = b - nA;
            const int t = nA + (h >> 1);
            gemm_tile<PAIR, TM / 2, NBW, VOUT>(c, (t % ntm) * TM + (h & 1) * (TM / 2), (t / ntm) * S::ROWS, g_lds);
            return;
        }
    }
    {
        const int t = b < nA ? b : b - (nH >> 1);
        gemm_tile<PAIR, TM, NBW, VOUT>(c, (t % ntm) * TM, (t / ntm) * S::ROWS, g_lds);
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

static int cu_count() { return device_cu_count(); }

template <bool PAIR, int TM, int NBW, bool VOUT>
hipError_t go_big(const Contract &c, hipStream_t s) {
    using S = GemmShape<PAIR, TM, NBW>;
    const int ntm = (c.M + TM - 1) / TM;
    const int ntn = (c.R + S::ROWS - 1) / S::ROWS;
    const int tiles = ntm * ntn;
    // Half tiles for the CUs' second workgroups when the grid holds at least
    // 2.5 tiles per CU, and only for plain outputs: the gate|up pair writes
    // half the bytes (ReLU^2 . up), and at M = 4096 the shifted launch took
    // 140 us against 128 us.
    const int cus = cu_count();
    const bool shift = !PAIR && TM % 64 == 0 && 2 * tiles >= 5 * cus;
    // nH half tiles pair up into whole tiles: it must be even (an odd count
    // would leave the second half of the last tile unwritten).
    const int nA = shift ? cus : tiles;
    const int nH = shift ? (cus & ~1) : 0;
    const size_t lds = (size_t)kGStages * S::STAGE;
    if (hipError_t e = allow_dynamic_lds((const void *)k_gemm_big<PAIR, TM, NBW, VOUT>, lds); e != hipSuccess)
        return e;
    hipLaunchKernelGGL((k_gemm_big<PAIR, TM, NBW, VOUT>), dim3(tiles + nH / 2), dim3(256), lds, s, c, ntm, nA, nH);
    return hipGetLastError();
}

// The vector-store epilogue writes 4 consecutive output columns per lane: every
// group of 4 packed rows (the columns of one field) must lie in one segment
// (segment sizes multiples of 4 packed rows), and the rows and base pointer
// must be aligned for 16-byte (fp32, int32) or 8-byte (bf16) stores.
static bool vout_ok(const Contract &c) {
    if (c.R % 4 != 0 || c.ldy % 4 != 0) return false;
    const size_t esz = c.y_dt == BL_BF16 ? 2 : 4;
    if ((uintptr_t)c.y % (4 * esz) != 0) return false;
    if (!c.pair)
        for (int i = 0; i <= c.seg.n; ++i)
            if (c.seg.roff[i] % 4 != 0) return false;
    return true;
}

template <bool PAIR, int TM, int NBW>
hipError_t go_big_v(const Contract &c, hipStream_t s) {
    return vout_ok(c) ? go_big<PAIR, TM, NBW, true>(c, s) : go_big<PAIR, TM, NBW, false>(c, s);
}

hipError_t launch_gemm(const Contract &c0, int *qsum_ws, hipStream_t s) {
    Contract c = c0;
    // Large tiles when K fits whole 128-byte stages and the grid still fills
    // the chip; the field scale of the masked unpack (x16) must not overflow.
    // (A 256-token tile needs 256 accumulator registers per lane, which the
    // compiler does not keep in the accumulator file: it copies them around
    // every MFMA.  128-token tiles keep all 128 in place.)
    // c.qsum already set: the quantizer wrote the row code sums.
    if ((c.qsum != nullptr || qsum_ws != nullptr) && c.K % kGK == 0 && c.ldq % 16 == 0 && c.K <= (1 << 18)) {
        if (c.qsum == nullptr) {
            hipLaunchKernelGGL(k_code_sums, dim3(c.M), dim3(256), 0, s, c.q, c.ldq, c.M, c.K, qsum_ws);
            if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
            c.qsum = qsum_ws;
        }
        // Tile shape: 128 or 96 tokens x 64 or 32 packed rows (the gate|up
        // pair: 32 + 32), whichever finishes first in a model of the launch:
        // rounds of two workgroups per CU, each round costing its tile's
        // work, a round with at most one workgroup per CU 0.6 of it, divided
        // by the shape's relative MFMA efficiency (smaller tiles reuse each
        // operand fragment fewer times).
        const int cus = cu_count();
        auto cost = [&](int tm, int rows, double eff) {
            const long tiles = (long)((c.M + tm - 1) / tm) * ((c.R + rows - 1) / rows);
            double t = 0.0;
            for (long left = tiles; left > 0; left -= 2L * cus)
                t += (double)tm * rows * (left > cus ? 1.0 : 0.6);
            return t / eff;
        };
        if (c.pair) {
            if (cost(96, 32, 0.95) < cost(128, 32, 1.0)) return go_big_v<true, 96, 2>(c, s);
            return go_big_v<true, 128, 2>(c, s);
        }
        const double cand[4] = {cost(128, 64, 1.0), cost(128, 32, 0.9), cost(96, 64, 0.95), cost(96, 32, 0.85)};
        int pick = 0;
        for (int i = 1; i < 4; ++i)
            if (cand[i] < cand[pick]) pick = i;
        switch (pick) {
        case 0: return go_big_v<false, 128, 2>(c, s);
        case 1: return go_big_v<false, 128, 1>(c, s);
        case 2: return go_big_v<false, 96, 2>(c, s);
        default: return go_big_v<false, 96, 1>(c, s);
        }
    }
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
