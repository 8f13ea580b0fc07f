// k_attn.hip -- the attention side of a decoder layer for one new token
// (decode): RoPE on the token's query and key, its key and value appended to
// the caches, and grouped-query softmax attention over every cached position
// and the token itself.
//
// "BitNet" model documentation, "模型详情" (rotary position embeddings) and
// "BitNetConfig" (20 attention heads, 5 key/value heads for grouped-query
// attention, hidden size 2560 = 20 heads x 128 dimensions, rope_theta as a
// parameter).  The rotation pairs dimension i of a head with i + 64 at angle
// pos * base^(-i/64); the scores are scaled by 1/sqrt(128).
//
// Two launches.  k_attn_partial: one workgroup per (key/value head, chunk of
// 64 positions); it reads each cached key and value of its chunk once, into
// registers, for all query heads of the group:
//   keys    thread (dg = t & 15, ps = t >> 4) holds dimensions 4dg..4dg+3 and
//           64+4dg..64+4dg+3 of positions ps, ps+16, ps+32, ps+48 (a 16-lane
//           row group reads a whole 512-byte row in two loads);
//   values  thread (dp = t & 63, pq = t >> 6) holds dimensions 2dp, 2dp+1 of
//           positions 16pq .. 16pq+15 (a wave reads a whole row per load).
// The rotated queries go through LDS; each thread forms its dimensions' part
// of the scores of its 4 positions for every head and the row group sums
// them (DPP reduce-scatter); one wave per head takes the maximum, the
// exponentials and their sum over the chunk; each thread accumulates its 16
// positions' weighted values for every head and the four position quarters
// meet in LDS.  The workgroup owning pos rotates the token's key, stores it
// and the value into the caches and uses them in place of its row.  Each
// chunk writes (max, sum, 128 partial outputs) per head to the workspace;
// k_attn_combine, one workgroup per query head, merges the chunks (weights
// exp(max_c - max)).  A single chunk (pos < 64) writes the output itself and
// the second launch is skipped.
// Everything is fp32.
#include "bl_common.h"

namespace bl {

namespace {

constexpr int kAttnD = 128;
constexpr int kAttnChunk = 64;
constexpr int kAttnMaxGroup = 4;                 // query heads per key/value head
constexpr int kAttnPart = kAttnD + 4;            // per head and chunk: max, sum, 2 unused, 128 outputs
constexpr int kAttnMaxChunks = 512;              // max_seq <= 32768

struct AttnArgs {
    const float *q, *k_new, *v_new;
    float *k_cache, *v_cache;
    const float *rcos, *rsin;   // [max_seq][64]
    float *part;                // [H][nchunks][kAttnPart]
    float *out;                 // [H][128]
    int pos, H, KVH, G, max_seq, nchunks;
    float scale;
};

// Lane exchanges within a 16-lane DPP row.
template <int Ctrl>
__device__ __forceinline__ float dpp_f(float v) {
    return __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), Ctrl, 0xF, 0xF, false));
}
constexpr int kDppQuadSwap1 = 0xB1;     // quad_perm(1,0,3,2): lane ^ 1
constexpr int kDppQuadSwap2 = 0x4E;     // quad_perm(2,3,0,1): lane ^ 2
constexpr int kDppHalfMirror = 0x141;   // lane ^ 7 within the row
constexpr int kDppMirror = 0x140;       // lane ^ 15 within the row

// Four per-lane values s[0..3] (one per query head) summed over the 16 lanes
// of a row, scattered: lane i of the row returns the sum of s[i >> 2].  Two
// halving exchanges (lane ^ 15, then lane ^ 7) each keep half the heads and
// send the other half; the quad then sums its four lanes.
__device__ __forceinline__ float row16_reduce_scatter4(const float s[4], int i) {
    const bool hi = (i & 8) != 0, hq = (i & 4) != 0;
    const float k0 = hi ? s[2] : s[0], k1 = hi ? s[3] : s[1];
    const float t0 = hi ? s[0] : s[2], t1 = hi ? s[1] : s[3];
    const float u0 = k0 + dpp_f<kDppMirror>(t0);
    const float u1 = k1 + dpp_f<kDppMirror>(t1);
    const float kk = hq ? u1 : u0, tt = hq ? u0 : u1;
    float v = kk + dpp_f<kDppHalfMirror>(tt);
    v = v + dpp_f<kDppQuadSwap1>(v);
    v = v + dpp_f<kDppQuadSwap2>(v);
    return v;
}

// Maximum and sum over a whole wave (every lane active): the row by DPP, the
// four rows through lane reads.
__device__ __forceinline__ float wave64_max(float v) {
    v = fmaxf(v, dpp_f<kDppQuadSwap1>(v));
    v = fmaxf(v, dpp_f<kDppQuadSwap2>(v));
    v = fmaxf(v, dpp_f<kDppHalfMirror>(v));
    v = fmaxf(v, dpp_f<kDppMirror>(v));
    const int b = __float_as_int(v);
    return fmaxf(fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 0)), __int_as_float(__builtin_amdgcn_readlane(b, 16))),
                 fmaxf(__int_as_float(__builtin_amdgcn_readlane(b, 32)), __int_as_float(__builtin_amdgcn_readlane(b, 48))));
}
__device__ __forceinline__ float wave64_sum(float v) {
    v = v + dpp_f<kDppQuadSwap1>(v);
    v = v + dpp_f<kDppQuadSwap2>(v);
    v = v + dpp_f<kDppHalfMirror>(v);
    v = v + dpp_f<kDppMirror>(v);
    const int b = __float_as_int(v);
    return (__int_as_float(__builtin_amdgcn_readlane(b, 0)) + __int_as_float(__builtin_amdgcn_readlane(b, 16))) +
           (__int_as_float(__builtin_amdgcn_readlane(b, 32)) + __int_as_float(__builtin_amdgcn_readlane(b, 48)));
}

__global__ __launch_bounds__(256) void k_attn_partial(AttnArgs a) {
    __shared__ float qs[kAttnMaxGroup][kAttnD];      // rotated queries
    __shared__ float sc[kAttnMaxGroup][kAttnChunk];  // scaled scores
    __shared__ float4 pw[kAttnChunk];                // probabilities, [position][head]
    __shared__ float2 red[4][kAttnMaxGroup][64];     // weighted values per position quarter
    __shared__ float knew[kAttnD], vnew[kAttnD];     // the token's rotated key and its value
    const int g = blockIdx.x;
    const int c = blockIdx.y;
    const int t = threadIdx.x;
    const int j0 = c * kAttnChunk;
    const int n = a.pos + 1 - j0 < kAttnChunk ? a.pos + 1 - j0 : kAttnChunk;   // valid rows (>= 1)
    const int jn = a.pos - j0;                                                  // the token's row, if < 64
    const float *cs = a.rcos + (size_t)a.pos * (kAttnD / 2);
    const float *sn = a.rsin + (size_t)a.pos * (kAttnD / 2);
    const float *kc = a.k_cache + (size_t)g * a.max_seq * kAttnD;
    const float *vc = a.v_cache + (size_t)g * a.max_seq * kAttnD;
    // Rows at or past pos are read from row pos - 1 instead (row 0 for an
    // empty cache): loaded, given no weight, and never the row this call writes.
    const int jmax = a.pos > 0 ? a.pos - 1 : 0;

    // every load first: queries and rotation (threads past the group read the
    // last head's), keys, values
    const int hq = min(t >> 6, a.G - 1), iq = t & 63;
    const float *qh = a.q + (size_t)(g * a.G + hq) * kAttnD;
    const float x0 = qh[iq], x1 = qh[iq + 64], co = cs[iq], si = sn[iq];
    const int dg = t & 15, ps = t >> 4;
    float4 kr[4][2];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const float *row = kc + (size_t)min(j0 + ps + 16 * i, jmax) * kAttnD;
        kr[i][0] = *reinterpret_cast<const float4 *>(row + 4 * dg);
        kr[i][1] = *reinterpret_cast<const float4 *>(row + 64 + 4 * dg);
    }
    const int dp = t & 63, pq = t >> 6;
    float2 vr[16];
#pragma unroll
    for (int i = 0; i < 16; ++i)
        vr[i] = *reinterpret_cast<const float2 *>(vc + (size_t)min(j0 + 16 * pq + i, jmax) * kAttnD + 2 * dp);

    qs[t >> 6][iq] = x0 * co - x1 * si;   // rows past the group hold copies no head reads
    qs[t >> 6][iq + 64] = x1 * co + x0 * si;
    if (jn < kAttnChunk) {   // the owner of pos: the token's rotated key and its value, also into the caches
        if (t < kAttnD / 2) {
            const float *kh = a.k_new + (size_t)g * kAttnD;
            const float y0 = kh[t] * cs[t] - kh[t + 64] * sn[t];
            const float y1 = kh[t + 64] * cs[t] + kh[t] * sn[t];
            knew[t] = y0;
            knew[t + 64] = y1;
            float *kw = a.k_cache + ((size_t)g * a.max_seq + a.pos) * kAttnD;
            kw[t] = y0;
            kw[t + 64] = y1;
        } else if (t < kAttnD) {
            const int d = t - 64;
            const float *vh = a.v_new + (size_t)g * kAttnD;
            vnew[d] = vh[d];
            vnew[d + 64] = vh[d + 64];
            float *vw = a.v_cache + ((size_t)g * a.max_seq + a.pos) * kAttnD;
            vw[d] = vh[d];
            vw[d + 64] = vh[d + 64];
        }
    }
    __syncthreads();
    if (jn < kAttnChunk) {
#pragma unroll
        for (int i = 0; i < 4; ++i)
            if (ps + 16 * i == jn) {
                kr[i][0] = *reinterpret_cast<const float4 *>(&knew[4 * dg]);
                kr[i][1] = *reinterpret_cast<const float4 *>(&knew[64 + 4 * dg]);
            }
#pragma unroll
        for (int i = 0; i < 16; ++i)
            if (16 * pq + i == jn) vr[i] = *reinterpret_cast<const float2 *>(&vnew[2 * dp]);
    }

    // scores: this thread's 8 dimensions of its 4 positions for every head
    // (fused multiply-adds), reduce-scattered over the row group so that lane
    // dg holds head dg >> 2's score; lanes of one quad store the same value
    float4 qa[kAttnMaxGroup][2];
#pragma unroll
    for (int h = 0; h < kAttnMaxGroup; ++h) {
        qa[h][0] = *reinterpret_cast<const float4 *>(&qs[h][4 * dg]);
        qa[h][1] = *reinterpret_cast<const float4 *>(&qs[h][64 + 4 * dg]);
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float sh[kAttnMaxGroup];
#pragma unroll
        for (int h = 0; h < kAttnMaxGroup; ++h) {
            float d = qa[h][0].x * kr[i][0].x;
            d = fmaf(qa[h][0].y, kr[i][0].y, d);
            d = fmaf(qa[h][0].z, kr[i][0].z, d);
            d = fmaf(qa[h][0].w, kr[i][0].w, d);
            d = fmaf(qa[h][1].x, kr[i][1].x, d);
            d = fmaf(qa[h][1].y, kr[i][1].y, d);
            d = fmaf(qa[h][1].z, kr[i][1].z, d);
            d = fmaf(qa[h][1].w, kr[i][1].w, d);
            sh[h] = d;
        }
        sc[dg >> 2][ps + 16 * i] = row16_reduce_scatter4(sh, dg) * a.scale;
    }
    __syncthreads();

    // softmax over the chunk: wave w for head w
    const int w = t >> 6, lane = t & 63;
    float mw = 0.0f, lw = 1.0f;   // wave w: head w's maximum and sum over the chunk
    if (w < a.G) {
        const float sv = lane < n ? sc[w][lane] : -INFINITY;
        mw = wave64_max(sv);
        const float p = lane < n ? expf(sv - mw) : 0.0f;
        lw = wave64_sum(p);
        reinterpret_cast<float *>(pw)[lane * 4 + w] = p;
    } else {
        reinterpret_cast<float *>(pw)[lane * 4 + w] = 0.0f;   // heads past the group
    }
    __syncthreads();

    // weighted values of this thread's 16 positions, every head
    float2 acc[kAttnMaxGroup];
#pragma unroll
    for (int h = 0; h < kAttnMaxGroup; ++h) acc[h] = make_float2(0.0f, 0.0f);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const float4 pv = pw[16 * pq + i];
        acc[0].x = fmaf(pv.x, vr[i].x, acc[0].x);
        acc[0].y = fmaf(pv.x, vr[i].y, acc[0].y);
        acc[1].x = fmaf(pv.y, vr[i].x, acc[1].x);
        acc[1].y = fmaf(pv.y, vr[i].y, acc[1].y);
        acc[2].x = fmaf(pv.z, vr[i].x, acc[2].x);
        acc[2].y = fmaf(pv.z, vr[i].y, acc[2].y);
        acc[3].x = fmaf(pv.w, vr[i].x, acc[3].x);
        acc[3].y = fmaf(pv.w, vr[i].y, acc[3].y);
    }
#pragma unroll
    for (int h = 0; h < kAttnMaxGroup; ++h) red[pq][h][dp] = acc[h];
    __syncthreads();
    if (w < a.G) {   // thread (head w, dimensions 2 lane, 2 lane + 1) sums the quarters
        float2 o = red[0][w][lane];
#pragma unroll
        for (int q4 = 1; q4 < 4; ++q4) {
            const float2 r = red[q4][w][lane];
            o.x = o.x + r.x;
            o.y = o.y + r.y;
        }
        if (a.nchunks == 1) {   // the only chunk: its normalized sum is the result
            a.out[(size_t)(g * a.G + w) * kAttnD + 2 * lane] = o.x / lw;
            a.out[(size_t)(g * a.G + w) * kAttnD + 2 * lane + 1] = o.y / lw;
        } else {
            float *pr = a.part + ((size_t)(g * a.G + w) * a.nchunks + c) * kAttnPart;
            if (lane == 0) {
                pr[0] = mw;
                pr[1] = lw;
            }
            *reinterpret_cast<float2 *>(pr + 4 + 2 * lane) = o;
        }
    }
}

constexpr int kCombWaves = 8;
constexpr int kCombBatch = 8;   // chunks a wave loads before it consumes any

// One workgroup per query head; wave w takes chunks w, w + 8, ... in batches
// of eight whose loads (max, sum, two outputs a lane) are all issued first,
// keeping a running maximum and rescaling what it holds when the maximum
// grows.  The eight waves' (max, sum, outputs) then meet in LDS.
__global__ __launch_bounds__(64 * kCombWaves) void k_attn_combine(AttnArgs a) {
    __shared__ float red[kCombWaves][kAttnPart];
    const int h = blockIdx.x;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63;
    const float *pr = a.part + (size_t)h * a.nchunks * kAttnPart;
    float Mw = -INFINITY, L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c0 = w; c0 < a.nchunks; c0 += kCombBatch * kCombWaves) {
        float mm[kCombBatch], ll[kCombBatch];
        float2 ov[kCombBatch];
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            const int c = c0 + i * kCombWaves;
            const float *pc = pr + (size_t)(c < a.nchunks ? c : c0) * kAttnPart;
            mm[i] = pc[0];
            ll[i] = pc[1];
            ov[i] = *reinterpret_cast<const float2 *>(pc + 4 + 2 * lane);
        }
        float mb = Mw;
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) mb = fmaxf(mb, mm[i]);
        const float r = expf(Mw - mb);   // 0 before the first batch
        L = L * r;
        o0 = o0 * r;
        o1 = o1 * r;
#pragma unroll
        for (int i = 0; i < kCombBatch; ++i) {
            // a slot past the last chunk re-read chunk c0: it leaves the
            // maximum unchanged and gets no weight
            const float e = c0 + i * kCombWaves < a.nchunks ? expf(mm[i] - mb) : 0.0f;
            L = L + e * ll[i];
            o0 = o0 + e * ov[i].x;
            o1 = o1 + e * ov[i].y;
        }
        Mw = mb;
    }
    red[w][2 + 2 * lane] = o0;
    red[w][3 + 2 * lane] = o1;
    if (lane == 0) {
        red[w][0] = Mw;
        red[w][1] = L;
    }
    __syncthreads();
    if (w != 0) return;
    float M = red[0][0];
#pragma unroll
    for (int i = 1; i < kCombWaves; ++i) M = fmaxf(M, red[i][0]);
    float sl = 0.0f, s0 = 0.0f, s1 = 0.0f;
#pragma unroll
    for (int i = 0; i < kCombWaves; ++i) {
        const float e = expf(red[i][0] - M);   // 0 for a wave without chunks
        sl = sl + e * red[i][1];
        s0 = s0 + e * red[i][2 + 2 * lane];
        s1 = s1 + e * red[i][3 + 2 * lane];
    }
    a.out[(size_t)h * kAttnD + 2 * lane] = s0 / sl;
    a.out[(size_t)h * kAttnD + 2 * lane + 1] = s1 / sl;
}

} // namespace

size_t attn_decode_workspace_bytes(int n_heads, int max_seq) {
    const int nch = (max_seq + kAttnChunk - 1) / kAttnChunk;
    return (size_t)n_heads * nch * kAttnPart * sizeof(float);
}

int attn_decode_max_seq() { return kAttnMaxChunks * kAttnChunk; }

hipError_t launch_attn_decode(const float *q, const float *k_new, const float *v_new, int pos, int H, int KVH,
                              float *k_cache, float *v_cache, int max_seq, const float *rcos, const float *rsin,
                              float *out, void *ws, hipStream_t s) {
    AttnArgs a;
    a.q = q; a.k_new = k_new; a.v_new = v_new;
    a.k_cache = k_cache; a.v_cache = v_cache;
    a.rcos = rcos; a.rsin = rsin;
    a.part = static_cast<float *>(ws);
    a.out = out;
    a.pos = pos; a.H = H; a.KVH = KVH; a.G = H / KVH; a.max_seq = max_seq;
    a.nchunks = (pos + 1 + kAttnChunk - 1) / kAttnChunk;
    a.scale = 1.0f / sqrtf((float)kAttnD);
    hipLaunchKernelGGL(k_attn_partial, dim3(KVH, a.nchunks), dim3(256), 0, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess || a.nchunks == 1) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(H), dim3(64 * kCombWaves), 0, s, a);
    return hipGetLastError();
}

} // namespace bl
