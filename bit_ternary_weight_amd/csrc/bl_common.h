// bl_common.h -- internal declarations shared by the libbitlinear HIP sources.
// Not part of the public ABI (that is include/bitlinear.h).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include <map>
#include <mutex>
#include <utility>

#include "bitlinear.h"

namespace bl {

// Compute units of the current device (queried once per device; 256 if the
// query fails).  Thread-safe.
inline int device_cu_count() {
    static std::mutex mu;
    static std::map<int, int> cus;
    int dev = 0;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return 256;
    }
    std::lock_guard<std::mutex> lock(mu);
    auto it = cus.find(dev);
    if (it != cus.end()) return it->second;
    int n = 0;
    if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess || n <= 0) {
        (void)hipGetLastError();
        n = 256;
    }
    cus[dev] = n;
    return n;
}

// Allows `bytes` of dynamic LDS for `kernel` on the current device (needed
// above 64 KiB): set once per (device, kernel) and raised when a launch needs
// more.  Thread-safe; a failure is returned and not left pending.
inline hipError_t allow_dynamic_lds(const void *kernel, size_t bytes) {
    static std::mutex mu;
    static std::map<std::pair<int, const void *>, size_t> allowed;
    int dev = 0;
    if (hipError_t e = hipGetDevice(&dev); e != hipSuccess) {
        (void)hipGetLastError();
        return e;
    }
    std::lock_guard<std::mutex> lock(mu);
    size_t &have = allowed[{dev, kernel}];
    if (have >= bytes) return hipSuccess;
    hipError_t e = hipFuncSetAttribute(kernel, hipFuncAttributeMaxDynamicSharedMemorySize, (int)bytes);
    if (e != hipSuccess) {
        (void)hipGetLastError();
        return e;
    }
    have = bytes;
    return hipSuccess;
}

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

// Static indices only (selects): a run-time index into the table would make
// the compiler copy a kernel argument into scratch memory.
__device__ __forceinline__ ColOf col_of(const SegTab &t, int rr, int f) {
    int s = 0, r0 = t.roff[0], r1 = t.roff[1];
#pragma unroll
    for (int i = 1; i < BL_MAX_SEGMENTS; ++i)
        if (i < t.n && rr >= t.roff[i]) {
            s = i;
            r0 = t.roff[i];
            r1 = t.roff[i + 1];
        }
    return ColOf{s, 4 * r0 + f * (r1 - r0) + (rr - r0)};
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

// Wave-wide reductions without LDS round trips: DPP within each 16-lane row
// (xor 1, xor 2, rotate 4, rotate 8 leave every lane of a row holding the
// row's result), then the four rows combined in order through readlane.  The
// result is uniform and its summation order fixed.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int v) {
    return __builtin_amdgcn_update_dpp(0, v, CTRL, 0xF, 0xF, false);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double v) {
    const long long b = __double_as_longlong(v);
    const int lo = dpp_i<CTRL>((int)(b & 0xFFFFFFFF));
    const int hi = dpp_i<CTRL>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

__device__ __forceinline__ double readlane_d(double v, int l) {
    const long long b = __double_as_longlong(v);
    const int lo = __builtin_amdgcn_readlane((int)(b & 0xFFFFFFFF), l);
    const int hi = __builtin_amdgcn_readlane((int)(b >> 32), l);
    return __longlong_as_double(((long long)hi << 32) | (unsigned int)lo);
}

// Sum over each quad of lanes (every lane of the quad gets the sum).
__device__ __forceinline__ int quad_sum(int v) {
    v += dpp_i<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_i<0x4E>(v);    // quad_perm [2,3,0,1]
    return v;
}

__device__ __forceinline__ int wave_sum_dpp(int v) {
    v += dpp_i<0xB1>(v);    // quad_perm [1,0,3,2]
    v += dpp_i<0x4E>(v);    // quad_perm [2,3,0,1]
    v += dpp_i<0x124>(v);   // row_ror:4
    v += dpp_i<0x128>(v);   // row_ror:8
    return __builtin_amdgcn_readlane(v, 0) + __builtin_amdgcn_readlane(v, 16) +
           __builtin_amdgcn_readlane(v, 32) + __builtin_amdgcn_readlane(v, 48);
}

__device__ __forceinline__ double wave_sum_dpp(double v) {
    v += dpp_d<0xB1>(v);
    v += dpp_d<0x4E>(v);
    v += dpp_d<0x124>(v);
    v += dpp_d<0x128>(v);
    return ((readlane_d(v, 0) + readlane_d(v, 16)) + readlane_d(v, 32)) + readlane_d(v, 48);
}

__device__ __forceinline__ float wave_max_dpp(float v) {
    v = fmaxf(v, __int_as_float(dpp_i<0xB1>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i<0x4E>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i<0x124>(__float_as_int(v))));
    v = fmaxf(v, __int_as_float(dpp_i<0x128>(__float_as_int(v))));
    const int iv = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(iv, 0)), __int_as_float(__builtin_amdgcn_readlane(iv, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(iv, 32)), __int_as_float(__builtin_amdgcn_readlane(iv, 48))));
}

// Workgroup barrier ordering LDS only: wait for this wave's LDS operations
// (lgkmcnt 0), then s_barrier.  __syncthreads() (and the compiler's own
// barrier lowering) would also wait for every outstanding global load of the
// wave, i.e. for a whole weight stream in flight.  The barrier is written as
// an asm statement with a memory clobber so no LDS access moves across it.
__device__ __forceinline__ void lds_barrier() {
    __builtin_amdgcn_s_waitcnt(0xC07F);   // lgkmcnt(0); vmcnt, expcnt unconstrained
    asm volatile("s_barrier" ::: "memory");
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

// Four consecutive outputs of one row from one lane (y 16-byte aligned for
// fp32 / int32, 8-byte for bf16; the values of int32 output are the exact
// accumulators carried as float bit patterns).
__device__ __forceinline__ void store4(void *y, int y_dt, size_t idx, const float v[4]) {
    if (y_dt == BL_F32) {
        *reinterpret_cast<float4 *>((float *)y + idx) = make_float4(v[0], v[1], v[2], v[3]);
    } else if (y_dt == BL_BF16) {
        const uint32_t lo = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
        const uint32_t hi = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
        *reinterpret_cast<uint2 *>((uint16_t *)y + idx) = make_uint2(lo, hi);
    } else {
        *reinterpret_cast<int4 *>((int32_t *)y + idx) =
            make_int4(__float_as_int(v[0]), __float_as_int(v[1]), __float_as_int(v[2]), __float_as_int(v[3]));
    }
}

// ReLU^2(gate) * up on already-rescaled fp32 values (two roundings, no FMA).
__device__ __forceinline__ float relu2_mul(float g, float u) {
    float gp = g > 0.0f ? g : 0.0f;
    float sq = gp * gp;
    return sq * u;
}

// ---------------------------------------------------------------------------
// int8 MFMA helpers shared by the contraction kernels.
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
// Operand layout of v_mfma_i32_16x16x64_i8: lane l supplies row (l & 15) of
// A and column (l & 15) of B, each as 16 int8 values of k-group (l >> 4); A
// and B use the same k placement, so any consistent assignment of k to
// (group, byte) gives the same dot products.  The 16x16 int32 result sits in
// lane l as rows 4*(l >> 4) + j, column l & 15, for j = 0..3.
// ---------------------------------------------------------------------------
typedef int v4i __attribute__((ext_vector_type(4)));

__device__ __forceinline__ v4i ld16(const void *p) { return *reinterpret_cast<const v4i *>(p); }

__device__ __forceinline__ v4i mfma16(v4i a, v4i b, v4i c) {
    return __builtin_amdgcn_mfma_i32_16x16x64_i8(a, b, c, 0, 0, 0);
}

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

// Output of one accumulator entry: packed row vr, field f, token row m with
// activation scale a.  PAIR: A is the gate accumulator, U the up one, and the
// output is ReLU^2(gate)*up at column f*R + vr.
__device__ __forceinline__ void emit_out(void *y, int y_dt, int ldy, bool pair, const SegTab &seg, int R,
                                         const float *w_mean, int m, int vr, int f, float a, int A, int U) {
    if (pair) {
        const float gv = (float)A * (w_mean[0] / a);
        const float uv = (float)U * (w_mean[1] / a);
        const float p = relu2_mul(gv, uv);
        const size_t idx = (size_t)m * ldy + f * R + vr;
        if (y_dt == BL_BF16)
            ((uint16_t *)y)[idx] = f32_to_bf16(p);
        else
            ((float *)y)[idx] = p;
    } else {
        const ColOf cs = col_of(seg, vr, f);
        store_out(y, y_dt, (size_t)m * ldy + cs.col, A, w_mean[cs.seg] / a);
    }
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
                            int *qsum, hipStream_t s);
// One per-token quantization (optionally preceded by RMSNorm): rows
// [0, M) of x (stride ldx) -> codes q (stride K), scales a, and, when qsum is
// not null, each row's code sum.
struct QuantProblem {
    const void *x;
    int8_t *q;
    float *a;
    int *qsum;          // [M] sum of the row's codes, or nullptr
    const float *gain;  // RMSNorm gain (nullptr: none)
    float eps;
    int norm;           // 1: RMSNorm before quantizing
    int x_dt, M, K, ldx, row0;
    int tile_m;         // 0: codes row-major [M,K]; else tiled, code_offset() with this token pitch
};
// Byte offset of code (m, k) in a code buffer: row-major [M,K] when tile_m is
// 0, else tiled by 64-byte pieces of K: piece k / 64 holds tile_m token rows
// of 64 codes each, so 16 tokens' codes of one piece are 1 KB contiguous.
__host__ __device__ inline size_t code_offset(int m, int k, int K, int tile_m) {
    return tile_m == 0 ? (size_t)m * K + k : ((size_t)(k >> 6) * tile_m + m) * 64 + (k & 63);
}

// Several row quantizations in one launch (the problems of a batched decode).
struct QuantBatch {
    int n;
    QuantProblem p[8];
};
hipError_t launch_quant_batch(QuantBatch &qb, hipStream_t s);
hipError_t launch_rmsnorm_quant(const void *h, int h_dt, int M, int K, const float *g, float eps,
                                int8_t *q, float *a, int *qsum, hipStream_t s);

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
    const int *qsum = nullptr;   // [M] code sums of the rows of q (nullptr: launch_gemm computes them)
};

// Decode path (M <= 64): one launch covers up to kMaxProblems independent
// contractions.  Modes: 0 = int8 codes in (x, a); 1 = raw fp32/bf16 x,
// quantized in the kernel's prologue; 2 = raw x, RMSNorm then quantized in
// the prologue.  Modes 1-2 need M <= kFuseMaxM and M*K <= kFuseMaxBytes.
constexpr int kMaxProblems = 8;
constexpr int kFuseMaxM = 4;
constexpr int kFuseMaxBytes = 48 * 1024;

struct GemvProblem {
    const void *x;      // mode 0: int8 codes; else fp32/bf16 activations
    const float *a;     // mode 0: activation scales [M]
    const float *gain;  // mode 2: RMSNorm gain [K] or null
    const uint8_t *P;   // packed weight, row stride K (PAIR: gate rows then up rows)
    const float *w_mean;
    void *y;
    int8_t *dbg_q;      // optional: the prologue's codes [M,K] (written once)
    float *dbg_a;       // optional: their scales [M]
    SegTab seg;
    int x_dt, ldx, M, K, R, y_dt, ldy, tile0, mode, pair;
    int cs;             // streaming variants: row groups per workgroup (4 rows; 16 in k_gemv_mt)
    float eps;
    const int *qsum;    // mode 0: the rows' code sums [M] when the quantizer wrote them, else null
    int qtile;          // mode 0: 0 = codes row-major with stride ldx; else tiled (code_offset) with this pitch
    int vout;           // k_gemv_mt: four consecutive packed rows land in four consecutive,
                        // 16-byte aligned output columns (vector stores)
};

struct GemvBatch {
    int n;
    int ring_off;   // LDS offset of the weight ring (streaming variant)
    GemvProblem p[kMaxProblems];
};

// Fills tile0 of every problem and launches; all problems must share `pair`.
hipError_t launch_gemv_batch(GemvBatch &b, hipStream_t s);
// Host check: decode problems with these M and K can go to the batched
// streaming kernel (k_gemv_mt), whose codes the quantizer then writes tiled.
bool gemv_mt_plan_ok(int n, const int *Ms, const int *Ks);
// Batched decode with tiled codes (k_gemv_mt.hip): every problem fits the
// kernel (tiled codes with their row sums, no gate|up pairing, K a multiple
// of 256, aligned operands), and its launch (hipErrorNotSupported when some
// problem's K needs more blocks per wave than the kernel holds).
bool gemv_mt_ok(const GemvBatch &b);
hipError_t launch_gemv_mt(GemvBatch &b, hipStream_t s);
// The batch's weight bytes (nb tensors per problem) divided evenly over cus
// workgroups: the per-workgroup budget the decode launchers size tiles by.
size_t even_share(const GemvBatch &b, int nb, int cus);
// Decode attention (k_attn.hip): workspace bytes (the per-chunk partial
// results for n_heads query heads over max_seq positions), the largest
// max_seq it serves, and the launches.
size_t attn_decode_workspace_bytes(int n_heads, int max_seq);
int attn_decode_max_seq();
hipError_t launch_attn_decode(const float *q, const float *k_new, const float *v_new, int pos, int H, int KVH,
                              float *k_cache, float *v_cache, int max_seq, const float *rcos, const float *rsin,
                              float *out, void *ws, hipStream_t s);
// Prefill GEMM (any M).  The large-tile kernel reads the rows' code sums
// instead of recomputing them per tile: from c.qsum when the caller has them,
// else computed into qsum_ws (device scratch for M ints); with neither the
// small-tile kernel runs.
hipError_t launch_gemm(const Contract &c, int *qsum_ws, hipStream_t s);

// Expired bounded waits counted by the decode kernels on the current device
// (synchronous read; reset clears the count).
hipError_t gemv_wait_expired(unsigned int *count, bool reset);
// Any K (slow, simple): used when K is not a multiple of 16.
hipError_t launch_generic(const Contract &c, hipStream_t s);

// The decode step of a stack of linear layers at one token in one
// persistent launch (k_chain.hip).
struct ChainLayerPtrs {
    const uint8_t *P_qkv;
    const float *w_qkv;
    const uint8_t *P_o;
    const float *w_o;
    const uint8_t *P_gu;
    const float *w_gu;
    const uint8_t *P_dn;
    const float *w_dn;
    const float *g_sub;
    const float *g_ffn;
};
struct ChainParams {
    const void *x;
    int x_dt;
    int L, H, KV, I;
    float eps;
    float *xch;      // [L][(H + 2KV) + H + I + H] fp32 exchange (packed-row order)
    float *stages;   // the same in column order, or null
    float *y;        // [H]
    int G;           // workgroups (chain_workgroups())
    SegTab seg_qkv;
    const ChainLayerPtrs *layers;   // host array of L
};
// The 1-bit BitLinear (k_binary.hip): one entry of a problem table.
struct W1Args {
    const void *x;        // raw activations [M, ldx] (fp32 or bf16), for the norm launch
    int x_dt, ldx;
    const float *gamma;   // [K] or null
    const float *beta;    // [K] or null
    int M, K;
    int8_t *q;            // [M, K] codes
    float *a;             // [M] activation scales
    const uint8_t *P;     // packed signs [N/8, K], for the contraction
    int N;
    const float *w_scale; // [1]
    float *y;             // [M, N] fp32
};
int w1_ln_max_k();
hipError_t launch_binarize_pack(const float *W, int N, int K, uint8_t *packed, hipStream_t s);
hipError_t launch_w1_norm(const W1Args *probs, int n, float eps, hipStream_t s);
hipError_t launch_w1_gemm(const W1Args *probs, int n, hipStream_t s);
bool w1_decode_fits(const W1Args *probs, int n);
hipError_t w1_wait_expired(unsigned int *count, bool reset);
hipError_t launch_w1_decode(const W1Args *probs, int n, float eps, hipStream_t s);

int chain_max_layers();
bool chain_fits(int H, int KV, int I, int G);
int chain_workgroups();
hipError_t launch_chain_decode(const ChainParams &p, hipStream_t s);
hipError_t chain_wait_expired(unsigned int *count, bool reset);

// Offline-unpacked weights (k_unpacked.hip): the packed weight expanded to
// bf16 codes W [N][K], and the decode-size product against it.
hipError_t launch_unpack_bf16(const uint8_t *packed, int N, int K, const SegTab &seg, void *w, hipStream_t s);

} // namespace bl
