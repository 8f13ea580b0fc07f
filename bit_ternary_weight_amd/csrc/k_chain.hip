// k_chain.hip -- the decode step of a whole stack of linear layers at one
// token (M = 1) in one persistent launch.
//
// Per layer (the BitNet model documentation, "模型详情" / "BitNetConfig":
// subln before the projections that follow attention and the FFN's ReLU^2;
// the article "Transformers 实战 BitNet 1.58 位量化", "推理侧 BitLinear" for
// each BitLinear), with attention left out as in the layer driver:
//   x -> quantize -> q|k|v            (three segments, one weight)
//     -> q quantize -> o
//     -> subln RMSNorm -> quantize -> gate|up -> ReLU^2(gate)*up
//     -> ffn_sub_norm RMSNorm -> quantize -> down -> next layer's x.
// Every BitLinear computes the same bits as the separate launches: per-token
// absmax codes, the integer contraction of the packed codes (kept as code+1,
// the code sum subtracted once), y = float(A) * (w_mean / a).
//
// Why one launch: each of the four stages needs the whole output vector of
// the previous one (a row maximum, a norm), so a layer is four dependent
// steps.  As separate launches every step paid a launch and a cold ramp of
// its weight stream.  Here the weights of a step do not wait for its input:
//
//   * one workgroup per compute unit (all resident; the host checks the
//     occupancy before launching), each owning a fixed set of 4-row groups of
//     every stage's weight;
//   * 12 stream waves hold the weight units (4 packed rows x 256 bytes) of a
//     stage in registers, loaded one stage ahead (issued as soon as the
//     previous stage's outputs have been stored), so a stage's weights do
//     not wait for its input.  They issue no other global memory operation,
//     so the compiler's waits on them stay exact;
//   * 4 quantizer waves poll the previous stage's output into LDS and reduce
//     its max |h| (and the norm's fp64 sum of squares) from the chunks they
//     hold; all 16 waves then normalize and quantize it; the stream waves add
//     each unit's products into one LDS accumulator per output, and the
//     quantizer waves, which formed the epilogue's constants meanwhile,
//     store this workgroup's part of the stage's output.
//
// Cross-workgroup exchange without fences or counters: every stage output
// goes to an exchange buffer that a fill launch sets to an all-ones word (a
// NaN no stage produces from finite input) right before the persistent
// launch.  The exchange holds a stage's outputs in packed-row order (output
// of packed row r, field f at 4 r + f), so a workgroup's outputs are one
// contiguous run of 64 or 128 bytes written by one store instruction, with
// agent-scope stores (the coherent cache policy); the column-order copy the
// caller may ask for is written with plain stores.  A consumer reads the
// vector with agent-scope loads until no word holds the fill pattern: each
// word is written once, so correctness rests on per-location coherence alone.
// Waits are bounded: an expired one is counted (bl_device_errors) and the
// kernel runs to its end.
//
// Within a workgroup the two roles meet at four barriers per stage (input in
// LDS; codes in LDS; products accumulated; outputs stored), all LDS-only so
// no wave waits for weight loads in flight.  The next stage's weights are
// issued after the last: a compute unit sends its memory requests in issue
// order, and stores queued behind a stage's worth of weight loads reach the
// other workgroups that much later.
#include "bl_buffer.h"
#include "bl_common.h"

namespace bl {

namespace {

constexpr int kCS = 12;                 // stream waves
constexpr int kCQ = 4;                  // quantizer / epilogue waves
constexpr int kCQL = kCQ * 64;
constexpr int kCWaves = kCS + kCQ;
constexpr int kCThreads = kCWaves * 64;
constexpr int kCMaxK = 8192;            // largest K: codes in LDS, polled words per lane
constexpr int kCUnit = 256;             // k bytes of a unit
// Weight units per stream wave and stage (q|k|v, o, gate|up, down): a
// workgroup owns at most 12 * kU units of a stage.
constexpr int kUq = 1, kUo = 1, kUg = 4, kUd = 3;
constexpr int kUMax = 4;
constexpr int kCMaxUnits = kCS * kUMax;
constexpr int kCMaxAcc = 2 * 4 * 16;    // outputs of a workgroup: 2 tensors x 4 groups x 16 (the host bounds ng)
constexpr unsigned kFill = 0xFFFFFFFFu;  // exchange words not yet written
constexpr int kPollMax = 1 << 17;       // polls per wait (each at least a memory round trip)

__device__ unsigned int g_chain_expired = 0;

struct ChainLayer {
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

constexpr int kChainMaxLayers = 32;

struct ChainArgs {
    const void *x;
    int x_dt;
    int L, H, KV, I;
    float eps;
    float *xch;      // [L][Sw] exchange, packed-row order: q|k|v, o, p, y
    float *stages;   // [L][Sw] the same in column order, or null
    int Sw;
    float *y;        // [H]
    int G;           // workgroups
    SegTab seg_qkv;
    ChainLayer layers[kChainMaxLayers];
};

// The launch's single argument, read through the kernel-argument pointer so
// that a run-time layer index is a scalar load, not a copy of the table.
__device__ __forceinline__ const ChainArgs &args() {
    return *(const ChainArgs *)__builtin_amdgcn_kernarg_segment_ptr();
}

// Stage geometry of this workgroup, the same for every layer: computed once.
struct Stage {
    const uint8_t *P;  // packed weight (pair: gate rows, then up rows)
    int K;             // input width (bytes of a packed row)
    int R;             // packed rows of one tensor
    int nt;            // tensors (2: gate|up)
    int g0, ng;        // this workgroup's 4-row groups [g0, g0 + ng)
    int ku;            // units along K
    int nunits;        // nt * ng * ku
};

// The launch-wide fields, read from the kernel arguments once, all together,
// at the start: left to itself the compiler issues each kernel-argument load
// next to its first use, so every stage's epilogue and next-stage issue
// waited on one dependent round trip after another.  The stage geometry is
// recomputed at each use from these (scalar arithmetic on uniform values)
// rather than kept: a table of it would be placed in scratch memory.
struct Geo {
    int L, H, KV, I, Sw, G, x_dt;
    float eps;
    float *xch, *stages, *y;
    const void *x;
    SegTab seg;
};

__device__ __forceinline__ Geo make_geo(const ChainArgs &A) {
    Geo g;
    g.L = A.L; g.H = A.H; g.KV = A.KV; g.I = A.I; g.Sw = A.Sw; g.G = A.G; g.x_dt = A.x_dt;
    g.eps = A.eps; g.xch = A.xch; g.stages = A.stages; g.y = A.y; g.x = A.x;
    g.seg = A.seg_qkv;
    asm volatile("" ::"s"(g.L), "s"(g.H), "s"(g.KV), "s"(g.I), "s"(g.Sw), "s"(g.G), "s"(g.x_dt), "s"(g.eps),
                 "s"(g.xch), "s"(g.stages), "s"(g.y), "s"(g.x));
#pragma unroll
    for (int i = 0; i <= BL_MAX_SEGMENTS; ++i) asm volatile("" ::"s"(g.seg.roff[i]));
    asm volatile("" ::"s"(g.seg.n));
    return g;
}

__device__ __forceinline__ Stage stage_of(const ChainArgs &A, const Geo &g, int l, int s) {
    const ChainLayer &w = A.layers[l];
    Stage st;
    if (s == 0) { st.P = w.P_qkv; st.K = g.H; st.R = (g.H + 2 * g.KV) / 4; st.nt = 1; }
    else if (s == 1) { st.P = w.P_o; st.K = g.H; st.R = g.H / 4; st.nt = 1; }
    else if (s == 2) { st.P = w.P_gu; st.K = g.H; st.R = g.I / 4; st.nt = 2; }
    else { st.P = w.P_dn; st.K = g.I; st.R = g.H / 4; st.nt = 1; }
    const int groups = st.R / 4;
    const int b = blockIdx.x;
    st.g0 = b * groups / g.G;
    st.ng = (b + 1) * groups / g.G - st.g0;
    st.ku = st.K / kCUnit;
    st.nunits = st.nt * st.ng * st.ku;
    return st;
}

// Global address of this lane's 16 bytes of unit mu (clamped to a valid unit;
// a workgroup with no group of this stage reads its neighbour's first unit).
// The lanes of a wave cover 4 packed rows x 256 bytes: lane (g, l) holds row
// l >> 2, chunk (l & 3) + 4g, the operand layout of the MFMA consumption.
__device__ __forceinline__ const uint8_t *unit_addr(const Stage &st, int mu, int lane) {
    int t = 0, gr = 0, k = 0;
    if (st.nunits > 0) {
        const int m = mu < st.nunits ? mu : st.nunits - 1;
        k = m % st.ku;
        const int rest = m / st.ku;
        gr = st.g0 + rest % st.ng;
        t = rest / st.ng;
    } else {
        gr = st.g0 < st.R / 4 ? st.g0 : st.R / 4 - 1;
    }
    const int row = t * st.R + 4 * gr + ((lane & 15) >> 2);
    const int ch = (lane & 3) + 4 * (lane >> 4);
    return st.P + (size_t)row * st.K + (size_t)k * kCUnit + 16 * ch;
}

template <int U>
__device__ __forceinline__ void issue(const Stage &st, int ws, int lane, v4i (&r)[U]) {
#pragma unroll
    for (int u = 0; u < U; ++u)
        r[u] = __builtin_nontemporal_load(reinterpret_cast<const v4i *>(unit_addr(st, ws + kCS * u, lane)));
}

// Consumes this wave's units of a stage: per unit, each field through one
// v_mfma_i32_16x16x64_i8 (weights first, the codes of the same chunks
// second), the k-slice sums of each row gathered from the quad that holds
// them; lane 16r adds the unit's 4 fields of unit row r into the row's
// accumulators acc[((tensor, group) * 4 + r) * 4 + field] (LDS integer
// atomics: exact and order-free), which the quantizer waves cleared.
// Row r's sum over its four k-slices, at lane 16 r of a quad: entry s of the
// product held by lane 16 r + s (quad broadcasts of lanes 1, 2, 3 of the quad;
// the other lanes' results are not used).
__device__ __forceinline__ int quad_diag(const v4i &d) {
    return d[0] + dpp_i<0x55>(d[1]) + dpp_i<0xAA>(d[2]) + dpp_i<0xFF>(d[3]);   // quad_perm [1,1,1,1] ...
}

template <int U>
__device__ __forceinline__ void consume(const Stage &st, int ws, int lane, const v4i (&r)[U], const int8_t *q_s,
                                        int *acc) {
    const int ch = (lane & 3) + 4 * (lane >> 4);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int mu = ws + kCS * u;
        if (mu >= st.nunits) break;
        const int k = mu % st.ku;
        const v4i b = *reinterpret_cast<const v4i *>(q_s + k * kCUnit + 16 * ch);
        v4i f[4];
        expand(r[u], f);
        int tot[4];
#pragma unroll
        for (int fi = 0; fi < 4; ++fi) {
            const v4i d = mfma16(f[fi], b, v4i{0, 0, 0, 0});
            tot[fi] = shift_field(quad_diag(d), fi);
        }
        if ((lane & 15) == 0) {
            int *dst = acc + ((mu / st.ku) * 4 + (lane >> 4)) * 4;
#pragma unroll
            for (int fi = 0; fi < 4; ++fi) atomicAdd(dst + fi, tot[fi]);
        }
    }
}

struct ChainLds {
    float xs[kCMaxK];            // the stage input, exchange order
    float xg[kCMaxK];            // its RMSNorm gains, exchange order
    int8_t q_s[kCMaxK];          // its codes, column order
    int acc[kCMaxAcc];           // output accumulators: [tensor, group][unit row][field]
    alignas(16) double qp_d[kCQ];  // per quantizer wave: sum of squares of its chunks (norm stages)
    alignas(16) float qp_m[kCQ];   // per quantizer wave: max |value| of its chunks
    float q_r, q_mx;             // the norm's r and the input's absmax (norm stages)
    float red_f[kCWaves];        // per-wave absolute maxima (norm with a gain)
    int red_i[kCWaves];          // per-wave code sums
};

// ---------------------------------------------------------------------------
// A stage's input, its normalization and its quantization.
//
// The quantizer waves poll the input vector (exchange order) as 16-byte
// chunks, chunk c = ql + 256 i holding positions 4c .. 4c+3 (packed row c,
// fields 0..3, i.e. columns f K/4 + c), and copy it to LDS; then all 16 waves
// normalize and quantize it, thread t taking chunks t and t + 1024, so that
// no single wave runs a long sequence of dependent instructions.
// ---------------------------------------------------------------------------
constexpr int kCChunks = kCMaxK / 4 / kCQL;        // polled chunks per quantizer lane, at most
constexpr int kCNormChunks = kCMaxK / 4 / kCThreads;   // chunks per thread in the quantization
constexpr int kSc1 = 16;   // cache-policy operand of a buffer load: agent scope (the sc1 bit)

// The quantizer waves' share of the input's reductions, taken from the
// values they already hold in registers: this wave's max |value| and (norm
// stages) its fp64 sum of squares, to qp_m / qp_d of quantizer wave ql / 64.
// Each lane sums its chunks in order, then the wave (DPP): a fixed order.
__device__ __forceinline__ void publish_partials(float hm, double ss, bool norm, int ql, ChainLds &sh) {
    hm = wave_max_dpp(hm);
    if (norm) ss = wave_sum_dpp(ss);
    if ((ql & 63) == 0) {
        sh.qp_m[ql >> 6] = hm;
        sh.qp_d[ql >> 6] = ss;
    }
}

// Polls the K-word input `in` until no word of this lane's chunks holds the
// fill pattern, then stores the chunks to xs (and the matching gains, or
// ones, to xg) and publishes the wave's partial reductions.  Agent-scope
// loads of one poll are all in flight together.  `live` turns false after an
// expired poll; later polls take what they find.
__device__ __forceinline__ void poll_to_lds(const float *in, int K, const float *gain, bool norm, int ql,
                                            ChainLds &sh, bool &live) {
    float *xs = sh.xs, *xg = sh.xg;
    const int nc = K >> 2;
    const int ni = (nc + kCQL - 1) / kCQL;
    if (gain) {
        // the gains of this lane's chunks, fetched ahead of the poll
        float g[kCChunks][4];
#pragma unroll
        for (int i = 0; i < kCChunks; ++i) {
            const int c = ql + kCQL * i;
#pragma unroll
            for (int f = 0; f < 4; ++f) g[i][f] = (i < ni && c < nc) ? gain[f * nc + c] : 1.0f;
        }
#pragma unroll
        for (int i = 0; i < kCChunks; ++i) {
            const int c = ql + kCQL * i;
            if (i < ni && c < nc) *reinterpret_cast<float4 *>(xg + 4 * c) = float4{g[i][0], g[i][1], g[i][2], g[i][3]};
        }
    }
    const __amdgpu_buffer_rsrc_t rs = buf_rsrc(in, K * 4);
    v4i u[kCChunks];
    for (int it = 0;; ++it) {
#pragma unroll
        for (int i = 0; i < kCChunks; ++i) {
            u[i] = v4i{0, 0, 0, 0};
            if (i < ni) u[i] = __builtin_amdgcn_raw_buffer_load_b128(rs, (ql + kCQL * i) * 16, 0, kSc1);
        }
        bool missing = false;
#pragma unroll
        for (int i = 0; i < kCChunks; ++i) {
            const bool fill = (unsigned)u[i][0] == kFill || (unsigned)u[i][1] == kFill ||
                              (unsigned)u[i][2] == kFill || (unsigned)u[i][3] == kFill;
            missing |= (ql + kCQL * i < nc) && fill;
        }
        if (!missing) break;
        if (!live || it >= kPollMax) {
            if (live) atomicAdd(&g_chain_expired, 1u);
            live = false;
            break;
        }
        __builtin_amdgcn_s_sleep(1);
    }
    float hm = 0.0f;
    double ss = 0.0;
#pragma unroll
    for (int i = 0; i < kCChunks; ++i) {
        const int c = ql + kCQL * i;
        if (i < ni && c < nc) {
            *reinterpret_cast<v4i *>(xs + 4 * c) = u[i];
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const float v = __int_as_float(u[i][f]);
                hm = fmaxf(hm, fabsf(v));
                if (norm) ss += (double)v * (double)v;
            }
        }
    }
    publish_partials(hm, ss, norm, ql, sh);
}

// The first layer's input x (the caller's fp32 or bf16 row, column order),
// stored to xs in exchange order, with the wave's max |x|; xg is unused
// (stage 0 has no norm).
__device__ __forceinline__ void load_x(const Geo &A, int ql, ChainLds &sh) {
    const int nc = A.H >> 2;
    float hm = 0.0f;
    for (int c = ql; c < nc; c += kCQL) {
        float t[4];
#pragma unroll
        for (int f = 0; f < 4; ++f) {
            const int k = f * nc + c;
            t[f] = A.x_dt == BL_BF16 ? bf16_to_f32(static_cast<const uint16_t *>(A.x)[k])
                                     : static_cast<const float *>(A.x)[k];
            hm = fmaxf(hm, fabsf(t[f]));
        }
        *reinterpret_cast<float4 *>(sh.xs + 4 * c) = float4{t[0], t[1], t[2], t[3]};
    }
    publish_partials(hm, 0.0, false, ql, sh);
}

// The four quantizer waves' partial sums, added in wave order.
__device__ __forceinline__ double sum4(const double *p) {
    const double2 *q = reinterpret_cast<const double2 *>(p);
    const double2 a = q[0], b = q[1];
    return ((a.x + a.y) + b.x) + b.y;
}

__device__ __forceinline__ float max4(const float *p) {
    const float4 x = *reinterpret_cast<const float4 *>(p);
    return fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w));
}

__device__ __forceinline__ float max16(const float *p) {
    const float4 *q = reinterpret_cast<const float4 *>(p);
    float m = 0.0f;
#pragma unroll
    for (int i = 0; i < kCWaves / 4; ++i) {
        const float4 x = q[i];
        m = fmaxf(m, fmaxf(fmaxf(x.x, x.y), fmaxf(x.z, x.w)));
    }
    return m;
}

// All 16 waves: normalizes (optionally) and quantizes the K values in xs:
// codes to q_s in column order, this wave's code sum to red_i[wave]; returns
// the activation scale.  Same arithmetic as the row kernel: fp64 sum of
// squares, r = float(1 / sqrt(ss / K + eps)), (h * r) * g (g = 1 without a
// gain), a = 127 / max(amax, 1e-5), q = clamp(rint(x * a)).  The sum of
// squares and max |h| come from the quantizer waves' partials (published
// before the barrier that put xs in LDS); the sums run in a fixed order (per
// lane over its chunks, the wave, then the four waves in order).
__device__ __forceinline__ float quantize_all(int K, bool norm, bool has_gain, float eps, ChainLds &sh, bool qwave) {
    const int t = threadIdx.x, wave = t >> 6;
    const int nc = K >> 2;
    float v[kCNormChunks][4];
#pragma unroll
    for (int i = 0; i < kCNormChunks; ++i) {
        const int c = t + kCThreads * i;
        const float4 x = c < nc ? *reinterpret_cast<const float4 *>(sh.xs + 4 * c) : float4{0.0f, 0.0f, 0.0f, 0.0f};
        v[i][0] = x.x; v[i][1] = x.y; v[i][2] = x.z; v[i][3] = x.w;
    }
    float mx = 0.0f;
    bool have_max = false;
    if (norm) {
        // r's fp64 chain (two divisions and a square root) runs in the
        // quantizer waves only, one per SIMD, and reaches the others through
        // LDS: sixteen waves repeating it would queue on the fp64 units
        if (qwave) {
            const float rq = (float)(1.0 / sqrt(sum4(sh.qp_d) / (double)K + (double)eps));
            // without a gain the largest |h * r| is float(max |h| * r): the
            // rounded product is monotone in the first factor and odd, so the
            // maximum commutes with it (one exchange saved)
            if (t == kCS * 64) {
                sh.q_r = rq;
                sh.q_mx = max4(sh.qp_m) * rq;
            }
        }
        lds_barrier();   // r in LDS
        const float r = sh.q_r;
        if (!has_gain) {
            mx = sh.q_mx;
            have_max = true;
        }
#pragma unroll
        for (int i = 0; i < kCNormChunks; ++i) {
            const int c = t + kCThreads * i;
            float4 g{1.0f, 1.0f, 1.0f, 1.0f};
            if (has_gain && c < nc) g = *reinterpret_cast<const float4 *>(sh.xg + 4 * c);
            v[i][0] = (v[i][0] * r) * g.x; v[i][1] = (v[i][1] * r) * g.y;
            v[i][2] = (v[i][2] * r) * g.z; v[i][3] = (v[i][3] * r) * g.w;
        }
    }
    if (!norm) {
        mx = max4(sh.qp_m);
        have_max = true;
    }
    if (!have_max) {
        float am = 0.0f;
#pragma unroll
        for (int i = 0; i < kCNormChunks; ++i)
#pragma unroll
            for (int f = 0; f < 4; ++f) am = fmaxf(am, fabsf(v[i][f]));
        am = wave_max_dpp(am);
        if ((t & 63) == 0) sh.red_f[wave] = am;
        lds_barrier();
        mx = max16(sh.red_f);
    }
    const float a = 127.0f / fmaxf(mx, 1e-5f);
    int cs = 0;
#pragma unroll
    for (int i = 0; i < kCNormChunks; ++i) {
        const int c = t + kCThreads * i;
        if (c < nc) {
#pragma unroll
            for (int f = 0; f < 4; ++f) {
                const int qi = (int)__builtin_amdgcn_fmed3f(rintf(v[i][f] * a), -128.0f, 127.0f);
                sh.q_s[f * nc + c] = (int8_t)qi;
                cs += qi;
            }
        }
    }
    cs = wave_sum_dpp(cs);
    if ((t & 63) == 0) sh.red_i[wave] = cs;
    return a;
}

// This workgroup's outputs of a stage: quantizer lane ql < 16 ng takes group
// ql / 16, row (ql / 4) % 4, field ql % 4: its row's accumulated sum less the
// code sum, then the rescale (and ReLU^2 for the pair).  Exchange position
// 4 rr + f = 16 g0 + ql: the lanes store one contiguous run, agent-scope (the
// next stage polls it); the column-order copies are plain stores.
//
// Everything but the sums is formed by ep_prepare while the stream waves
// multiply (the scale and code sums are known once the codes are): after the
// last barrier only a subtraction, a conversion, a multiply and the stores
// remain.  The rescale is float(A) * (w_mean / a), with IEEE fp32 division.
struct EpPrep {
    bool on;       // this lane stores an output
    int acc0;      // its accumulator (first tensor); acc1 the second (pair)
    int acc1;
    int qsum;      // the stage's code sum
    float s0, s1;  // w_mean / a of its segment (pair: gate, up)
    int col;       // column-order index
    int xo;        // exchange index
};

__device__ __forceinline__ EpPrep ep_prepare(const Geo &A, const Stage &st, int s, int ql, int qsum, float a,
                                             const float (&wm)[3]) {
    EpPrep e;
    e.on = ql < 16 * st.ng;
    const int grl = ql >> 4, row = (ql >> 2) & 3, f = ql & 3;
    e.acc0 = ((0 * st.ng + grl) * 4 + row) * 4 + f;
    e.acc1 = ((1 * st.ng + grl) * 4 + row) * 4 + f;
    e.qsum = qsum;
    const int rr = 4 * (st.g0 + grl) + row;   // packed row within its tensor
    e.s1 = 0.0f;
    if (s == 2) {
        e.s0 = wm[0] / a;
        e.s1 = wm[1] / a;
        e.col = f * st.R + rr;
    } else if (s == 0) {
        const ColOf c = col_of(A.seg, rr, f);
        e.s0 = (c.seg == 0 ? wm[0] : (c.seg == 1 ? wm[1] : wm[2])) / a;
        e.col = c.col;
    } else {
        e.s0 = wm[0] / a;
        e.col = f * st.R + rr;
    }
    e.xo = 16 * st.g0 + ql;
    return e;
}

__device__ __forceinline__ void ep_store(const EpPrep &e, int s, const int *accs, float *xout, float *out,
                                         float *y_last) {
    if (!e.on) return;
    const int A0 = accs[e.acc0] - e.qsum;
    float val;
    if (s == 2) {
        const int A1 = accs[e.acc1] - e.qsum;
        val = relu2_mul((float)A0 * e.s0, (float)A1 * e.s1);
    } else {
        val = (float)A0 * e.s0;
    }
    __hip_atomic_store(reinterpret_cast<unsigned *>(xout) + e.xo, __float_as_uint(val), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
    if (out) out[e.col] = val;
    if (y_last) y_last[e.col] = val;
}

// Offset of stage s's output (q|k|v, o, p, y) within a layer's row of the
// exchange and stage buffers.
__device__ __forceinline__ int stage_off(const Geo &A, int s) {
    return s == 0 ? 0 : (s == 1 ? A.H + 2 * A.KV : (s == 2 ? 2 * A.H + 2 * A.KV : 2 * A.H + 2 * A.KV + A.I));
}

__device__ __forceinline__ int stage_k(const Geo &A, int s) { return s == 3 ? A.I : A.H; }

__device__ __forceinline__ const float *stage_gain(const ChainArgs &A, int l, int s) {
    return s == 2 ? A.layers[l].g_sub : (s == 3 ? A.layers[l].g_ffn : nullptr);
}

// Stage s of layer l for the quantizer waves: input to LDS, barrier, the
// shared quantization, barrier (codes), barrier (partial sums), outputs,
// barrier (outputs stored).
__device__ __forceinline__ void q_stage(const ChainArgs &A, const Geo &geo, int l, int s, int ql, ChainLds &sh,
                                        bool &live) {
    const Stage st = stage_of(A, geo, l, s);
    float *xl = geo.xch + (size_t)l * geo.Sw;
    const int K = stage_k(geo, s);
    const float *gain = stage_gain(A, l, s);
    float wm[3] = {1.0f, 1.0f, 1.0f};
    {
        // the epilogue's weight scales, fetched ahead of the wait
        const ChainLayer &w = A.layers[l];
        if (s == 0) { wm[0] = w.w_qkv[0]; wm[1] = w.w_qkv[1]; wm[2] = w.w_qkv[2]; }
        else if (s == 1) wm[0] = w.w_o[0];
        else if (s == 2) { wm[0] = w.w_gu[0]; wm[1] = w.w_gu[1]; }
        else wm[0] = w.w_dn[0];
    }
    asm volatile("" ::"s"(gain));
    // the output accumulators start at zero (the previous stage's epilogue
    // read them before its last barrier)
    for (int i = ql; i < kCMaxAcc; i += kCQL) sh.acc[i] = 0;
    if (s == 0 && l == 0) {
        load_x(geo, ql, sh);
    } else {
        const float *in = s == 0 ? xl - geo.Sw + stage_off(geo, 3) : xl + stage_off(geo, s - 1);
        poll_to_lds(in, K, gain, s >= 2, ql, sh, live);
    }
    lds_barrier();   // input in LDS
    const float a = quantize_all(K, s >= 2, gain != nullptr, geo.eps, sh, true);
    lds_barrier();   // codes ready
    // while the stream waves multiply: the epilogue's constants
    int qsum = 0;
#pragma unroll
    for (int w = 0; w < kCWaves; ++w) qsum += sh.red_i[w];
    const EpPrep ep = ep_prepare(geo, st, s, ql, qsum, a, wm);
    const int so = stage_off(geo, s);
    float *out = geo.stages ? geo.stages + (size_t)l * geo.Sw + so : nullptr;
    float *y_last = (s == 3 && l == geo.L - 1) ? geo.y : nullptr;
    lds_barrier();   // products accumulated
    ep_store(ep, s, sh.acc, xl + so, out, y_last);
    lds_barrier();   // outputs stored: the next stage's weights may queue behind them
}

// The stream waves' registers: one set of unit slots per stage kind.
struct Ring {
    v4i q[kUq], o[kUo], g[kUg], d[kUd];
};

// Stage S of layer l for the stream waves: the shared quantization, the
// products, and then the next stage's weights, issued after the outputs have
// been stored (requests leave a compute unit in issue order: stores queued
// behind a stage of weight loads would reach the consumers that much later).
// The weights land during the next stage's poll and quantization.
template <int S>
__device__ __forceinline__ void s_stage(const ChainArgs &A, const Geo &geo, int l, int ws, int lane, Ring &rg,
                                        ChainLds &sh) {
    const Stage st = stage_of(A, geo, l, S);
    constexpr int NS = (S + 1) & 3;
    // the next stage's weight pointer and this stage's gain pointer read
    // before the first barrier, not where they are used
    const bool more = !(S == 3 && l + 1 >= geo.L);
    const uint8_t *nP = nullptr;
    if (more) {
        const ChainLayer &wn = A.layers[S == 3 ? l + 1 : l];
        nP = NS == 0 ? wn.P_qkv : (NS == 1 ? wn.P_o : (NS == 2 ? wn.P_gu : wn.P_dn));
    }
    const float *gp = stage_gain(A, l, S);
    asm volatile("" ::"s"(nP), "s"(gp));
    const bool has_gain = gp != nullptr;
    lds_barrier();   // input in LDS
    (void)quantize_all(stage_k(geo, S), S >= 2, has_gain, geo.eps, sh, false);
    lds_barrier();   // codes ready
    if (S == 0) consume<kUq>(st, ws, lane, rg.q, sh.q_s, sh.acc);
    if (S == 1) consume<kUo>(st, ws, lane, rg.o, sh.q_s, sh.acc);
    if (S == 2) consume<kUg>(st, ws, lane, rg.g, sh.q_s, sh.acc);
    if (S == 3) consume<kUd>(st, ws, lane, rg.d, sh.q_s, sh.acc);
    lds_barrier();   // products accumulated
    lds_barrier();   // outputs stored
    if (!more) return;   // no stage follows the last one
    Stage nx = stage_of(A, geo, S == 3 ? l + 1 : l, NS);
    nx.P = nP;
    if (NS == 0) issue<kUq>(nx, ws, lane, rg.q);
    if (NS == 1) issue<kUo>(nx, ws, lane, rg.o);
    if (NS == 2) issue<kUg>(nx, ws, lane, rg.g);
    if (NS == 3) issue<kUd>(nx, ws, lane, rg.d);
}

__global__ __launch_bounds__(kCThreads) void k_chain_decode(ChainArgs a_unused) {
    (void)a_unused;
    const ChainArgs &A = args();
    __shared__ __attribute__((aligned(16))) ChainLds sh;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)), lane = threadIdx.x & 63;
    const Geo geo = make_geo(A);
    if (wave < kCS) {
        Ring rg;
        issue<kUq>(stage_of(A, geo, 0, 0), wave, lane, rg.q);
        for (int l = 0; l < geo.L; ++l) {
            s_stage<0>(A, geo, l, wave, lane, rg, sh);
            s_stage<1>(A, geo, l, wave, lane, rg, sh);
            s_stage<2>(A, geo, l, wave, lane, rg, sh);
            s_stage<3>(A, geo, l, wave, lane, rg, sh);
        }
    } else {
        const int ql = threadIdx.x - kCS * 64;
        bool live = true;
#pragma unroll 1
        for (int i = 0; i < 4 * geo.L; ++i) q_stage(A, geo, i >> 2, i & 3, ql, sh, live);
    }
}

// Sets every word of the exchange buffers to the fill pattern.
__global__ __launch_bounds__(256) void k_chain_fill(unsigned *p, size_t n) {
    for (size_t i = (size_t)blockIdx.x * 256 + threadIdx.x; i < n; i += (size_t)gridDim.x * 256) p[i] = kFill;
}

} // namespace

int chain_max_layers() { return kChainMaxLayers; }

// Host check of the shapes against the kernel's fixed capacities (units per
// stream wave and stage, output accumulators, LDS codes) for G workgroups.
bool chain_fits(int H, int KV, int I, int G) {
    if (H % kCUnit || I % kCUnit || KV % 16 || H > kCMaxK || I > kCMaxK || G < 1) return false;
    bool ok = true;
    auto units = [&](int R, int nt, int K) {
        const int groups = R / 4;
        const int per = (groups + G - 1) / G;
        if (nt * per * 16 > kCMaxAcc) ok = false;
        return nt * per * (K / kCUnit);
    };
    const bool fit = units((H + 2 * KV) / 4, 1, H) <= kCS * kUq && units(H / 4, 1, H) <= kCS * kUo &&
                     units(I / 4, 2, H) <= kCS * kUg && units(H / 4, 1, I) <= kCS * kUd;
    return fit && ok;
}

hipError_t launch_chain_decode(const ChainParams &p, hipStream_t s) {
    ChainArgs a{};
    a.x = p.x; a.x_dt = p.x_dt; a.L = p.L; a.H = p.H; a.KV = p.KV; a.I = p.I; a.eps = p.eps;
    a.xch = p.xch; a.stages = p.stages; a.Sw = (p.H + 2 * p.KV) + p.H + p.I + p.H; a.y = p.y; a.G = p.G;
    a.seg_qkv = p.seg_qkv;
    for (int l = 0; l < p.L; ++l) {
        const ChainLayerPtrs &w = p.layers[l];
        a.layers[l] = ChainLayer{w.P_qkv, w.w_qkv, w.P_o, w.w_o, w.P_gu, w.w_gu, w.P_dn, w.w_dn, w.g_sub, w.g_ffn};
    }
    const size_t words = (size_t)p.L * a.Sw;
    hipLaunchKernelGGL(k_chain_fill, dim3(256), dim3(256), 0, s, reinterpret_cast<unsigned *>(p.xch), words);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_chain_decode, dim3(p.G), dim3(kCThreads), 0, s, a);
    return hipGetLastError();
}

// Workgroups one launch may use: one per compute unit when the kernel fits
// one per unit (all resident at once, as the polls require), else 0.
int chain_workgroups() {
    const int cus = device_cu_count();
    int per = 0;
    if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per, reinterpret_cast<const void *>(&k_chain_decode), kCThreads,
                                                     0) != hipSuccess) {
        (void)hipGetLastError();
        return 0;
    }
    return per >= 1 ? cus : 0;
}

hipError_t chain_wait_expired(unsigned int *count, bool reset) {
    unsigned int v = 0;
    if (hipError_t e = hipMemcpyFromSymbol(&v, HIP_SYMBOL(g_chain_expired), sizeof(v)); e != hipSuccess) return e;
    if (reset && v) {
        const unsigned int zero = 0;
        if (hipError_t e = hipMemcpyToSymbol(HIP_SYMBOL(g_chain_expired), &zero, sizeof(zero)); e != hipSuccess)
            return e;
    }
    *count = v;
    return hipSuccess;
}

} // namespace bl
