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
// 64 positions).  It brings the chunk's keys and values into LDS with whole-
// row loads (the new token's row from its rotated key and its value, which
// the workgroup owning that position also stores into the caches), rotates
// the group's queries, and per query head (one wave each) forms the 64
// scores (a lane per position), their maximum, the exponentials and their
// sum, then the weighted value sum (a lane per two dimensions).  It writes
// (max, sum, 128 partial outputs) per head and chunk.  k_attn_combine: one
// wave per query head merges the chunks (rescaling each by exp(max_c - max)).
// Everything is fp32.
#include "bl_common.h"

namespace bl {

namespace {

constexpr int kAttnD = 128;
constexpr int kAttnChunk = 64;
constexpr int kAttnMaxGroup = 4;                 // query heads per key/value head
constexpr int kAttnKStride = kAttnD + 4;         // padded key rows: float4 reads of 64 rows spread over the banks
constexpr int kAttnPart = kAttnD + 2;            // per head and chunk: max, sum, 128 outputs

struct AttnArgs {
    const float *q, *k_new, *v_new;
    float *k_cache, *v_cache;
    const float *rcos, *rsin;   // [max_seq][64]
    float *part;                // [H][nchunks][kAttnPart]
    float *out;                 // [H][128]
    int pos, H, KVH, G, max_seq, nchunks;
    float scale;
};

__global__ __launch_bounds__(256) void k_attn_partial(AttnArgs a) {
    extern __shared__ __attribute__((aligned(16))) float sm[];
    float *Ks = sm;                                   // [64][kAttnKStride]
    float *Vs = Ks + kAttnChunk * kAttnKStride;       // [64][128]
    float *qs = Vs + kAttnChunk * kAttnD;             // [G][128]
    float *ps = qs + kAttnMaxGroup * kAttnD;          // [G][64]
    const int g = blockIdx.x;
    const int c = blockIdx.y;
    const int t = threadIdx.x;
    const int j0 = c * kAttnChunk;
    const int n = a.pos + 1 - j0 < kAttnChunk ? a.pos + 1 - j0 : kAttnChunk;   // valid rows (>= 1)
    const float *cs = a.rcos + (size_t)a.pos * (kAttnD / 2);
    const float *sn = a.rsin + (size_t)a.pos * (kAttnD / 2);

    // the group's rotated queries
    if (t < a.G * (kAttnD / 2)) {
        const int h = t >> 6, i = t & 63;
        const float *qh = a.q + (size_t)(g * a.G + h) * kAttnD;
        const float x0 = qh[i], x1 = qh[i + 64], co = cs[i], si = sn[i];
        qs[h * kAttnD + i] = x0 * co - x1 * si;
        qs[h * kAttnD + i + 64] = x1 * co + x0 * si;
    }
    // the chunk's keys and values (whole 512-byte rows, 32 lanes per row)
    float *kc = a.k_cache + (size_t)g * a.max_seq * kAttnD;
    float *vc = a.v_cache + (size_t)g * a.max_seq * kAttnD;
#pragma unroll
    for (int r = 0; r < 8; ++r) {
        const int idx = t + 256 * r;
        const int row = idx >> 5, c4 = idx & 31;
        const int j = j0 + row;
        float4 kv = make_float4(0.0f, 0.0f, 0.0f, 0.0f), vv = kv;
        if (j < a.pos) {
            kv = *reinterpret_cast<const float4 *>(kc + (size_t)j * kAttnD + 4 * c4);
            vv = *reinterpret_cast<const float4 *>(vc + (size_t)j * kAttnD + 4 * c4);
        }
        *reinterpret_cast<float4 *>(Ks + row * kAttnKStride + 4 * c4) = kv;
        *reinterpret_cast<float4 *>(Vs + row * kAttnD + 4 * c4) = vv;
    }
    // the new token's row: its rotated key and its value, also into the caches
    const int jn = a.pos - j0;
    if (jn < kAttnChunk) {
        __syncthreads();   // its row of the staging above is overwritten here
        if (t < kAttnD / 2) {
            const float *kh = a.k_new + (size_t)g * kAttnD;
            const float x0 = kh[t], x1 = kh[t + 64], co = cs[t], si = sn[t];
            const float y0 = x0 * co - x1 * si, y1 = x1 * co + x0 * si;
            Ks[jn * kAttnKStride + t] = y0;
            Ks[jn * kAttnKStride + t + 64] = y1;
            kc[(size_t)a.pos * kAttnD + t] = y0;
            kc[(size_t)a.pos * kAttnD + t + 64] = y1;
        } else if (t < kAttnD) {
            const int d = t - 64;
            const float *vh = a.v_new + (size_t)g * kAttnD;
            Vs[jn * kAttnD + d] = vh[d];
            Vs[jn * kAttnD + d + 64] = vh[d + 64];
            vc[(size_t)a.pos * kAttnD + d] = vh[d];
            vc[(size_t)a.pos * kAttnD + d + 64] = vh[d + 64];
        }
    }
    __syncthreads();

    const int w = t >> 6, lane = t & 63;
    if (w >= a.G) return;
    // scores of head w: lane = position
    float s = -INFINITY;
    if (lane < n) {
        const float4 *kr = reinterpret_cast<const float4 *>(Ks + lane * kAttnKStride);
        const float4 *qr = reinterpret_cast<const float4 *>(qs + w * kAttnD);
        float acc = 0.0f;
#pragma unroll 8
        for (int d4 = 0; d4 < kAttnD / 4; ++d4) {
            const float4 kk = kr[d4], qq = qr[d4];
            acc = acc + qq.x * kk.x;
            acc = acc + qq.y * kk.y;
            acc = acc + qq.z * kk.z;
            acc = acc + qq.w * kk.w;
        }
        s = acc * a.scale;
    }
    const float m = wave_max(s);
    const float p = lane < n ? expf(s - m) : 0.0f;
    float l = p;
#pragma unroll
    for (int o = 32; o > 0; o >>= 1) l += __shfl_xor(l, o, 64);
    ps[w * kAttnChunk + lane] = p;   // read back by this wave only: LDS operations of a wave complete in order
    __builtin_amdgcn_wave_barrier();
    // weighted values: lane = dimensions 2 lane, 2 lane + 1
    float o0 = 0.0f, o1 = 0.0f;
    for (int j = 0; j < n; ++j) {
        const float pj = ps[w * kAttnChunk + j];
        const float2 vv = *reinterpret_cast<const float2 *>(Vs + j * kAttnD + 2 * lane);
        o0 = o0 + pj * vv.x;
        o1 = o1 + pj * vv.y;
    }
    float *pr = a.part + ((size_t)(g * a.G + w) * a.nchunks + c) * kAttnPart;
    if (lane == 0) {
        pr[0] = m;
        pr[1] = l;
    }
    pr[2 + 2 * lane] = o0;
    pr[3 + 2 * lane] = o1;
}

__global__ __launch_bounds__(64) void k_attn_combine(AttnArgs a) {
    const int h = blockIdx.x;
    const int lane = threadIdx.x;
    const float *pr = a.part + (size_t)h * a.nchunks * kAttnPart;
    float M = -INFINITY;
    for (int c = 0; c < a.nchunks; ++c) M = fmaxf(M, pr[(size_t)c * kAttnPart]);
    float L = 0.0f, o0 = 0.0f, o1 = 0.0f;
    for (int c = 0; c < a.nchunks; ++c) {
        const float *pc = pr + (size_t)c * kAttnPart;
        const float e = expf(pc[0] - M);
        L = L + e * pc[1];
        o0 = o0 + e * pc[2 + 2 * lane];
        o1 = o1 + e * pc[3 + 2 * lane];
    }
    a.out[(size_t)h * kAttnD + 2 * lane] = o0 / L;
    a.out[(size_t)h * kAttnD + 2 * lane + 1] = o1 / L;
}

} // namespace

size_t attn_decode_part_bytes(int n_heads, int max_seq) {
    const int nch = (max_seq + kAttnChunk - 1) / kAttnChunk;
    return (size_t)n_heads * nch * kAttnPart * sizeof(float);
}

hipError_t launch_attn_decode(const float *q, const float *k_new, const float *v_new, int pos, int H, int KVH,
                              float *k_cache, float *v_cache, int max_seq, const float *rcos, const float *rsin,
                              float *out, float *part, hipStream_t s) {
    AttnArgs a;
    a.q = q; a.k_new = k_new; a.v_new = v_new;
    a.k_cache = k_cache; a.v_cache = v_cache;
    a.rcos = rcos; a.rsin = rsin;
    a.part = part; a.out = out;
    a.pos = pos; a.H = H; a.KVH = KVH; a.G = H / KVH; a.max_seq = max_seq;
    a.nchunks = (pos + 1 + kAttnChunk - 1) / kAttnChunk;
    a.scale = 1.0f / sqrtf((float)kAttnD);
    const size_t lds = sizeof(float) * ((size_t)kAttnChunk * kAttnKStride + (size_t)kAttnChunk * kAttnD +
                                        (size_t)kAttnMaxGroup * kAttnD + (size_t)kAttnMaxGroup * kAttnChunk);
    static bool attr = false;
    if (!attr) {
        if (hipError_t e = hipFuncSetAttribute(reinterpret_cast<const void *>(&k_attn_partial),
                                               hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds);
            e != hipSuccess)
            return e;
        attr = true;
    }
    hipLaunchKernelGGL(k_attn_partial, dim3(KVH, a.nchunks), dim3(256), lds, s, a);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_attn_combine, dim3(H), dim3(64), 0, s, a);
    return hipGetLastError();
}

} // namespace bl
