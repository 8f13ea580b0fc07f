// k_attn_prefill.hip -- the attention side of a decoder layer for a prompt
// of M tokens at positions 0 .. M-1 (prefill): RoPE on every token's query
// and key, the keys and values stored into the caches (for the decode steps
// that follow), and causal grouped-query softmax attention.
//
// "BitNet" model documentation, "模型详情" (rotary position embeddings) and
// "BitNetConfig" (20 attention heads, 5 key/value heads, hidden size 2560 =
// 20 heads x 128 dimensions, rope_theta a parameter).  The rotation pairs
// dimension i of a head with i + 64 at angle pos * base^(-i/64); scores are
// scaled by 1/sqrt(128); token p attends to positions 0 .. p.
//
// Two launches.
//   k_attn_prep: per 64 tokens and one head slot, the rotated queries and
//     keys rounded to bf16 (and the keys in fp32 into the cache), the values
//     into the cache and, rounded to bf16, transposed to [dimension][token].
//   k_attn_fwd: one workgroup per (query head, block of 128 queries),
//     heaviest blocks first; wave w owns two tiles of 16 queries, so every
//     key and value operand read from LDS feeds two products.  Per block of
//     64 keys
//     (staged through LDS, the next block's loads in flight meanwhile):
//       S^T = K Q^T  with v_mfma_f32_16x16x32_bf16 (keys the first operand,
//         so lane (g, c) holds keys 4g..4g+3 of each 16-key tile for query c);
//       online softmax in fp32 (base-2 exponentials of the pre-scaled
//         scores), the maximum shared by the four lanes of a query (lane
//         swaps) and moved
//         only when a block's exceeds it by more than 8;
//       O^T += V^T P^T with the probabilities rounded to bf16 straight from
//         the score registers: the k index of the product runs over the keys
//         in the order the score layout holds them, and the transposed value
//         block is read in the same order.
//     The result O^T / l is stored with 16-byte fp32 stores (four consecutive
//     dimensions of one query per lane).
#include "bl_common.h"
#include "bl_attn.h"

namespace bl {

namespace {

constexpr int kPD = 128;                 // head dimension
constexpr int kPB = 64;                  // tokens per key block (and per block of the prep kernel)
constexpr int kQT = 2;                   // 16-query tiles per wave
constexpr int kPQ = 4 * 16 * kQT;        // queries per workgroup (4 waves)
// LDS key rows of 128 bf16 (256 bytes, 16 pieces of 16), unpadded: piece p of
// row r sits at position p ^ (r & 15).  Lane group g of k-step s takes the
// dimensions of piece (g & 1) | s << 1 | (g >> 1) << 3 (a permutation of the
// dimension order that the queries share), so the 16 lanes of a group, and
// lanes l and l + 32, read distinct banks.
__device__ __forceinline__ int q_piece(int g, int s) { return (g & 1) | (s << 1) | ((g >> 1) << 3); }
constexpr int kVStride = kPB + 4;        // LDS transposed value row, bf16 elements (136 bytes)

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef __bf16 bf16x4 __attribute__((ext_vector_type(4)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

struct PrefArgs {
    const float *q, *k, *v;   // token rows with stride ldx: q head h at h*128, k / v head g at g*128
    int ldx;
    float *k_cache, *v_cache; // [KVH][max_seq][128]
    int max_seq;
    const float *rcos, *rsin; // [>= M][64]
    __bf16 *qb;               // [H][Mp][128] rotated queries
    __bf16 *kb;               // [KVH][Mp][128] rotated keys
    __bf16 *vt;               // [KVH][128][Mp] values, transposed
    float *out;               // [M][ldo]: head h at h*128
    int ldo;
    int M, Mp, H, KVH, G;
    float scale_log2;         // log2(e) / sqrt(128)
};

// bf16 of an fp32 value, rounded to nearest even (finite inputs).
__device__ __forceinline__ __bf16 to_bf(float x) { return static_cast<__bf16>(x); }

__global__ __launch_bounds__(256) void k_attn_prep(PrefArgs a) {
    __shared__ float vtile[kPB][kPD + 1];
    const int m0 = blockIdx.x * kPB;
    const int slot = blockIdx.y;          // < H: query head; < H + KVH: key head; else value head
    const int t = threadIdx.x;
    if (slot < a.H + a.KVH) {
        const bool isq = slot < a.H;
        const int hh = isq ? slot : slot - a.H;
        const float *src = (isq ? a.q : a.k) + hh * kPD;
        __bf16 *dst = (isq ? a.qb : a.kb) + (size_t)hh * a.Mp * kPD;
        const int i = t & 63;
#pragma unroll 4
        for (int r = 0; r < kPB / 4; ++r) {
            const int m = m0 + (t >> 6) + 4 * r;
            float y0 = 0.0f, y1 = 0.0f;
            if (m < a.M) {
                const float x0 = src[(size_t)m * a.ldx + i], x1 = src[(size_t)m * a.ldx + i + 64];
                const float co = a.rcos[(size_t)m * 64 + i], si = a.rsin[(size_t)m * 64 + i];
                y0 = x0 * co - x1 * si;
                y1 = x1 * co + x0 * si;
                if (!isq) {
                    float *kw = a.k_cache + ((size_t)hh * a.max_seq + m) * kPD;
                    kw[i] = y0;
                    kw[i + 64] = y1;
                }
            }
            dst[(size_t)m * kPD + i] = to_bf(y0);
            dst[(size_t)m * kPD + i + 64] = to_bf(y1);
        }
        return;
    }
    const int g = slot - a.H - a.KVH;
    const float *src = a.v + g * kPD;
#pragma unroll 4
    for (int r = 0; r < kPB / 2; ++r) {
        const int tok = (t >> 7) + 2 * r, d = t & 127;
        const int m = m0 + tok;
        float x = 0.0f;
        if (m < a.M) {
            x = src[(size_t)m * a.ldx + d];
            a.v_cache[((size_t)g * a.max_seq + m) * kPD + d] = x;
        }
        vtile[tok][d] = x;
    }
    __syncthreads();
    // transposed: thread (d = t >> 1, half = t & 1) writes 32 tokens of row d
    const int d = t >> 1, h0 = (t & 1) * 32;
    __bf16 *row = a.vt + ((size_t)g * kPD + d) * a.Mp + m0 + h0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        bf16x8 v8;
#pragma unroll
        for (int j = 0; j < 8; ++j) v8[j] = to_bf(vtile[h0 + 8 * c + j][d]);
        *reinterpret_cast<bf16x8 *>(row + 8 * c) = v8;
    }
}

// Maximum / sum over the four lanes l, l ^ 16, l ^ 32, l ^ 48 (a query's four
// lane groups), through the lane-swap instructions: swapping a register with
// itself returns the values of lanes l & ~16 and l | 16 (then l & ~32 and
// l | 32) in every lane.
__device__ __forceinline__ float group4_max(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = fmaxf(__uint_as_float(a[0]), __uint_as_float(a[1]));
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return fmaxf(__uint_as_float(b[0]), __uint_as_float(b[1]));
}
__device__ __forceinline__ float group4_sum(float v) {
    const auto a = __builtin_amdgcn_permlane16_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    v = __uint_as_float(a[0]) + __uint_as_float(a[1]);
    const auto b = __builtin_amdgcn_permlane32_swap(__float_as_uint(v), __float_as_uint(v), false, false);
    return __uint_as_float(b[0]) + __uint_as_float(b[1]);
}

// Row of the transposed value block that staging piece c (8 pieces a row)
// belongs to.  The 32 pieces c = 32k .. 32k+31 cover rows a, a+1, a+16, a+17
// (a from k), whose 8-byte halves, 136 bytes a row, fill all 32 bank pairs
// once: the LDS writes of lanes 0-31 do not conflict.
__device__ __forceinline__ int v_row(int c) {
    const int k = c >> 5, rs = (c >> 3) & 3;
    return (rs & 1) | ((rs >> 1) << 4) | ((k & 7) << 1) | ((k >> 3) << 5);
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// Two workgroups a CU: the register budget is held to 256 a lane (no spills).
__global__ __launch_bounds__(256) __attribute__((amdgpu_waves_per_eu(2, 2))) void k_attn_fwd(PrefArgs a) {
    __shared__ __attribute__((aligned(16))) __bf16 ks[kPB * kPD];
    __shared__ __attribute__((aligned(16))) __bf16 vs[kPD * kVStride];
    const int nqb = a.Mp / kPQ;
    const int qblk = nqb - 1 - (int)blockIdx.x / a.H;   // heaviest (latest) query blocks first
    const int h = (int)blockIdx.x % a.H;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, lr = lane & 15;
    const int kvh = h / a.G;
    int qrow[kQT];                                       // this lane's queries (positions), one per tile
#pragma unroll
    for (int u = 0; u < kQT; ++u) qrow[u] = qblk * kPQ + 16 * (kQT * w + u) + lr;
    const __bf16 *kbase = a.kb + (size_t)kvh * a.Mp * kPD;
    const __bf16 *vbase = a.vt + (size_t)kvh * kPD * a.Mp;

    // second operands of S^T = K Q^T: Q[query lr of tile u][the 8 dimensions
    // of piece q_piece(g, s)]
    bf16x8 qf[kQT][4];
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
        const __bf16 *qp = a.qb + ((size_t)h * a.Mp + qrow[u]) * kPD;
#pragma unroll
        for (int s = 0; s < 4; ++s) qf[u][s] = *reinterpret_cast<const bf16x8 *>(qp + 8 * q_piece(g, s));
    }
    // staging: 1024 16-byte pieces of keys (row c >> 4, piece c & 15) and of
    // transposed values (row v_row(c), piece c & 7), four of each per thread
    bf16x8 kr[4], vr[4];
    auto fetch = [&](int kb0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = t + 256 * r;
            kr[r] = *reinterpret_cast<const bf16x8 *>(kbase + (size_t)(kb0 + (c >> 4)) * kPD + 8 * (c & 15));
            vr[r] = *reinterpret_cast<const bf16x8 *>(vbase + (size_t)v_row(c) * a.Mp + kb0 + 8 * (c & 7));
        }
    };
    f32x4 o[kQT][8];
    float m_run[kQT], l_run[kQT];   // l_run: this lane's part (its keys) of the sum
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
        m_run[u] = -INFINITY;
        l_run[u] = 0.0f;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) o[u][dt] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    }
    const int nkb = (qblk + 1) * (kPQ / kPB);   // key blocks up to the last query of the block
    const int kdiag = qblk * (kPQ / kPB);       // key blocks from here on can hold keys past a query
    fetch(0);
    for (int kblk = 0; kblk < nkb; ++kblk) {
        __syncthreads();   // every wave is done with the previous block
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int c = t + 256 * r;
            *reinterpret_cast<bf16x8 *>(&ks[(c >> 4) * kPD + 8 * ((c & 15) ^ ((c >> 4) & 15))]) = kr[r];
            bf16x4 *vd = reinterpret_cast<bf16x4 *>(&vs[v_row(c) * kVStride + 8 * (c & 7)]);
            vd[0] = bf16x4{vr[r][0], vr[r][1], vr[r][2], vr[r][3]};
            vd[1] = bf16x4{vr[r][4], vr[r][5], vr[r][6], vr[r][7]};
        }
        __syncthreads();
        if (kblk + 1 < nkb) fetch((kblk + 1) * kPB);

        // S^T for 4 tiles of 16 keys, each key operand read once for both
        // query tiles: lane (g, lr) gets keys 16c + 4g + i of query lr
        f32x4 sc[kQT][4];
#pragma unroll
        for (int c = 0; c < 4; ++c) {
#pragma unroll
            for (int u = 0; u < kQT; ++u) sc[u][c] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
            for (int s = 0; s < 4; ++s) {
                const bf16x8 kf = *reinterpret_cast<const bf16x8 *>(&ks[(16 * c + lr) * kPD + 8 * (q_piece(g, s) ^ lr)]);
#pragma unroll
                for (int u = 0; u < kQT; ++u) sc[u][c] = mfma_bf16(kf, qf[u][s], sc[u][c]);
            }
        }
        bf16x8 pb[kQT][2];
#pragma unroll
        for (int u = 0; u < kQT; ++u) {
            // online softmax in base 2 (scores pre-scaled by log2(e)/sqrt(128))
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) sc[u][c][i] *= a.scale_log2;
            if (kblk >= kdiag) {   // blocks that reach past some query: those keys get no weight
#pragma unroll
                for (int c = 0; c < 4; ++c)
#pragma unroll
                    for (int i = 0; i < 4; ++i)
                        if (kblk * kPB + 16 * c + 4 * g + i > qrow[u]) sc[u][c][i] = -INFINITY;
            }
            float bm = -INFINITY;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) bm = fmaxf(bm, sc[u][c][i]);
            bm = group4_max(bm);
            // The running maximum moves only when a block's exceeds it by more
            // than 8 (so every weight stays below 2^8, well inside bf16 and
            // fp32); the accumulators are rescaled only then, which after the
            // first blocks is rare.  A block wholly past the query (-inf) never
            // moves it: every query has seen key 0 in block 0.
            const bool upd = bm > m_run[u] + 8.0f;
            if (__any(upd)) {
                const float m_new = upd ? bm : m_run[u];
                const float alpha = __builtin_amdgcn_exp2f(m_run[u] - m_new);   // 0 for the first block
                m_run[u] = m_new;
                l_run[u] *= alpha;
#pragma unroll
                for (int dt = 0; dt < 8; ++dt) o[u][dt] *= alpha;
            }
            float ps = 0.0f;
#pragma unroll
            for (int c = 0; c < 4; ++c)
#pragma unroll
                for (int i = 0; i < 4; ++i) {
                    const float p = __builtin_amdgcn_exp2f(sc[u][c][i] - m_run[u]);
                    ps += p;
                    pb[u][c >> 1][4 * (c & 1) + i] = to_bf(p);
                }
            l_run[u] += ps;
        }
        // O^T += V^T P^T: k slot 8g + j of step s is key 32s + 4g + j (j < 4)
        // or 32s + 16 + 4g + (j - 4); each value operand read once for both tiles
#pragma unroll
        for (int dt = 0; dt < 8; ++dt)
#pragma unroll
            for (int s = 0; s < 2; ++s) {
                const __bf16 *vrow = &vs[(16 * dt + lr) * kVStride + 32 * s + 4 * g];
                const bf16x4 lo = *reinterpret_cast<const bf16x4 *>(vrow);
                const bf16x4 hi = *reinterpret_cast<const bf16x4 *>(vrow + 16);
                const bf16x8 va = {lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
#pragma unroll
                for (int u = 0; u < kQT; ++u) o[u][dt] = mfma_bf16(va, pb[u][s], o[u][dt]);
            }
    }
#pragma unroll
    for (int u = 0; u < kQT; ++u) {
        const float l = group4_sum(l_run[u]);
        if (qrow[u] >= a.M) continue;
        const float inv = 1.0f / l;
        float *orow = a.out + (size_t)qrow[u] * a.ldo + h * kPD + 4 * g;
#pragma unroll
        for (int dt = 0; dt < 8; ++dt) {
            float4 v;
            v.x = o[u][dt][0] * inv;
            v.y = o[u][dt][1] * inv;
            v.z = o[u][dt][2] * inv;
            v.w = o[u][dt][3] * inv;
            *reinterpret_cast<float4 *>(orow + 16 * dt) = v;
        }
    }
}

} // namespace

size_t attn_prefill_workspace_bytes(int M, int n_heads, int n_kv_heads) {
    const size_t Mp = (size_t)(M + kPQ - 1) / kPQ * kPQ;
    return Mp * kPD * sizeof(__bf16) * ((size_t)n_heads + 2 * (size_t)n_kv_heads);
}

hipError_t launch_attn_prefill(const float *q, const float *k, const float *v, int ldx, int M, int H, int KVH,
                               float *k_cache, float *v_cache, int max_seq, const float *rcos, const float *rsin,
                               float *out, int ldo, void *ws, hipStream_t s) {
    PrefArgs a;
    a.q = q; a.k = k; a.v = v; a.ldx = ldx;
    a.k_cache = k_cache; a.v_cache = v_cache; a.max_seq = max_seq;
    a.rcos = rcos; a.rsin = rsin;
    a.M = M; a.Mp = (M + kPQ - 1) / kPQ * kPQ; a.H = H; a.KVH = KVH; a.G = H / KVH;
    a.qb = static_cast<__bf16 *>(ws);
    a.kb = a.qb + (size_t)H * a.Mp * kPD;
    a.vt = a.kb + (size_t)KVH * a.Mp * kPD;
    a.out = out; a.ldo = ldo;
    a.scale_log2 = 1.4426950408889634f / sqrtf((float)kPD);
    hipLaunchKernelGGL(k_attn_prep, dim3(a.Mp / kPB, H + 2 * KVH), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_fwd, dim3(a.Mp / kPQ * H), dim3(256), 0, s, a);
    return hipGetLastError();
}

} // namespace bl
