// k_unpacked.hip -- the offline-unpacked BitLinear: the packed ternary
// weight expanded once to dense bf16 codes, then the forward as a dense bf16
// product.  Article "Transformers 实战 BitNet 1.58 位量化", "BitNetQuantConfig"
// (AutoBitLinear with the offline mode: the packed weight is unpacked to the
// module's compute dtype when it is loaded, and the weight scale multiplies
// the output at inference) and "推理侧 BitLinear" (the unpack: field i under
// the mask 3 << 2i, minus 1).  The "BitNet" model documentation's note that
// the stock path brings no speed-up is what this path measures against the
// packed kernels.
//
// The activations are quantized per token as in the packed path and the
// codes enter the product as bf16 (exact), against the bf16 codes
// {-1, 0, 1} (exact).  Every product is an integer of magnitude <= 128 and
// every partial sum an integer below 2^24, so the fp32 sums are exact and the
// rescaled output is bit-identical to the packed path's.
//
//   k_unpack_bf16: W[n][k] = code(n, k) from the plane-order packed bytes
//     (within each stacked segment, packed row r, field f holds the
//     segment's weight row f*R_s + r); one thread per 16-byte piece of a
//     packed row, four output rows of 16 codes each.
//   k_gemv_bf16<MB>: decode rows (MB <= 4 token rows per launch pass): one
//     wave per weight row, 16-byte weight loads all issued before use, the
//     codes of the token rows as bf16 in LDS, v_dot2_f32_bf16 products; then
//     the BitLinear rescale.
// Prefill sizes use the bf16 MFMA GEMM of k_ste.hip with the BitLinear
// epilogue.
#include "bl_common.h"
#include "bl_ste.h"

namespace bl {

namespace {

typedef short s16x2 __attribute__((ext_vector_type(2)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));

// Packed row rr of a segmented weight (segments stacked along the packed
// rows, each packed on its own) holds, in field f, weight row
// 4 roff[s] + f R_s + (rr - roff[s]) of its segment s.
__global__ __launch_bounds__(256) void k_unpack_bf16(const uint8_t *P, int Rt, int K, SegTab seg, uint16_t *W) {
    const int per_row = (K + 15) / 16;
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    if (e >= (size_t)Rt * per_row) return;
    const int rr = (int)(e / per_row), k0 = (int)(e % per_row) * 16;
    const uint8_t *src = P + (size_t)rr * K + k0;
    uint8_t b[16];
    if (k0 + 16 <= K && ((uintptr_t)src & 15) == 0) {
        const uint4 v = *reinterpret_cast<const uint4 *>(src);
        const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = (uint8_t)(w[i >> 2] >> (8 * (i & 3)));
    } else {
#pragma unroll
        for (int i = 0; i < 16; ++i) b[i] = k0 + i < K ? src[i] : (uint8_t)0x55;
    }
#pragma unroll
    for (int f = 0; f < 4; ++f) {
        uint16_t *dst = W + (size_t)col_of(seg, rr, f).col * K + k0;
        uint16_t c[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int code = (int)((b[i] >> (2 * f)) & 3u) - 1;       // -1, 0, 1
            c[i] = code == 0 ? 0 : (code > 0 ? 0x3F80 : 0xBF80);      // bf16 of the code
        }
        if (k0 + 16 <= K && ((uintptr_t)dst & 15) == 0) {
            uint4 lo, hi;
            lo.x = c[0] | (uint32_t)c[1] << 16; lo.y = c[2] | (uint32_t)c[3] << 16;
            lo.z = c[4] | (uint32_t)c[5] << 16; lo.w = c[6] | (uint32_t)c[7] << 16;
            hi.x = c[8] | (uint32_t)c[9] << 16; hi.y = c[10] | (uint32_t)c[11] << 16;
            hi.z = c[12] | (uint32_t)c[13] << 16; hi.w = c[14] | (uint32_t)c[15] << 16;
            reinterpret_cast<uint4 *>(dst)[0] = lo;
            reinterpret_cast<uint4 *>(dst)[1] = hi;
        } else {
            for (int i = 0; i < 16; ++i)
                if (k0 + i < K) dst[i] = c[i];
        }
    }
}

constexpr int kGvWaves = 4;            // one weight row per wave
constexpr int kGvMaxK = 8192;          // codes staged in LDS: MB x K bf16
constexpr int kGvChunks = kGvMaxK / 8 / 64;   // 16-byte weight pieces per lane, at most

struct GvArgs {
    const int8_t *q;   // [M][K] activation codes
    const float *a;    // [M] scales
    const uint16_t *W; // [N][K] bf16 codes
    const float *w_mean;
    void *y;
    int M, K, N, ldy, y_dt, nseg;
    int cend[BL_MAX_SEGMENTS];
};

__device__ __forceinline__ float dot8(uint4 w, uint4 x, float acc) {
    const uint32_t ww[4] = {w.x, w.y, w.z, w.w}, xx[4] = {x.x, x.y, x.z, x.w};
#pragma unroll
    for (int i = 0; i < 4; ++i)
        acc = __builtin_amdgcn_fdot2_f32_bf16(__builtin_bit_cast(bf16x2, ww[i]), __builtin_bit_cast(bf16x2, xx[i]), acc,
                                              false);
    return acc;
}

// Token rows m0 .. m0 + MB - 1 (fewer at the end); each wave one weight row.
template <int MB>
__global__ __launch_bounds__(kGvWaves * 64) void k_gemv_bf16(GvArgs g, int m0) {
    __shared__ __attribute__((aligned(16))) uint16_t xs[MB * kGvMaxK];
    const int t = threadIdx.x, lane = t & 63, w = t >> 6;
    const int K = g.K, nm = min(MB, g.M - m0);
    // codes of the token rows as bf16 (zero rows past nm)
#pragma unroll
    for (int m = 0; m < MB; ++m) {
        const int *qrow = reinterpret_cast<const int *>(g.q + (size_t)(m0 + (m < nm ? m : 0)) * K);
        for (int k4 = t; k4 < K / 4; k4 += kGvWaves * 64) {
            const int v = m < nm ? qrow[k4] : 0;
            uint2 o;
            o.x = (__float_as_uint((float)(int8_t)(v & 0xFF)) >> 16) |
                  (__float_as_uint((float)(int8_t)((v >> 8) & 0xFF)) & 0xFFFF0000u);
            o.y = (__float_as_uint((float)(int8_t)((v >> 16) & 0xFF)) >> 16) |
                  (__float_as_uint((float)(int8_t)((v >> 24) & 0xFF)) & 0xFFFF0000u);
            *reinterpret_cast<uint2 *>(&xs[m * K + 4 * k4]) = o;
        }
    }
    const int n = blockIdx.x * kGvWaves + w;
    const int nch = K / 8;                       // whole 16-byte pieces (K % 8 == 0)
    uint4 wr[kGvChunks];
    const uint16_t *wrow = g.W + (size_t)(n < g.N ? n : g.N - 1) * K;
#pragma unroll
    for (int c = 0; c < kGvChunks; ++c) {
        const int ch = lane + 64 * c;
        wr[c] = ch < nch ? *reinterpret_cast<const uint4 *>(wrow + 8 * ch) : uint4{0, 0, 0, 0};
    }
    __syncthreads();
    float acc[MB];
#pragma unroll
    for (int m = 0; m < MB; ++m) acc[m] = 0.0f;
#pragma unroll
    for (int c = 0; c < kGvChunks; ++c) {
        const int ch = lane + 64 * c;
        if (ch < nch) {
#pragma unroll
            for (int m = 0; m < MB; ++m)
                acc[m] = dot8(wr[c], *reinterpret_cast<const uint4 *>(&xs[m * K + 8 * ch]), acc[m]);
        }
    }
#pragma unroll
    for (int m = 0; m < MB; ++m)
#pragma unroll
        for (int o = 32; o > 0; o >>= 1) acc[m] += __shfl_xor(acc[m], o, 64);
    if (lane != 0 || n >= g.N) return;
    int sg = 0;
#pragma unroll
    for (int s = 0; s < BL_MAX_SEGMENTS - 1; ++s) sg += (s + 1 < g.nseg && n >= g.cend[s]) ? 1 : 0;
    for (int m = 0; m < nm; ++m) {
        const size_t o = (size_t)(m0 + m) * g.ldy + n;
        const float v = acc[m] * (g.w_mean[sg] / g.a[m0 + m]);
        if (g.y_dt == BL_I32) static_cast<int *>(g.y)[o] = (int)acc[m];
        else if (g.y_dt == BL_BF16) static_cast<uint16_t *>(g.y)[o] = f32_to_bf16(v);
        else static_cast<float *>(g.y)[o] = v;
    }
}

} // namespace

hipError_t launch_unpack_bf16(const uint8_t *packed, int N, int K, const SegTab &seg, void *w, hipStream_t s) {
    const int R = N / 4;
    const size_t threads = (size_t)R * ((K + 15) / 16);
    hipLaunchKernelGGL(k_unpack_bf16, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, packed, R, K, seg,
                       static_cast<uint16_t *>(w));
    return hipGetLastError();
}

bool unpacked_gemv_fits(int K) { return K % 8 == 0 && K <= kGvMaxK; }

hipError_t launch_unpacked_gemv(const int8_t *q, const float *a, int M, int K, const void *W, int N, const GemmEpi &e,
                                void *y, hipStream_t s) {
    GvArgs g;
    g.q = q; g.a = a; g.W = static_cast<const uint16_t *>(W); g.w_mean = e.w_mean; g.y = y;
    g.M = M; g.K = K; g.N = N; g.ldy = N; g.y_dt = e.y_dt; g.nseg = e.nseg;
    for (int i = 0; i < BL_MAX_SEGMENTS; ++i) g.cend[i] = e.cend[i];
    const dim3 grid((N + kGvWaves - 1) / kGvWaves), block(kGvWaves * 64);
    for (int m0 = 0; m0 < M; m0 += 4) {
        const int nm = M - m0;
        if (nm >= 4) hipLaunchKernelGGL(k_gemv_bf16<4>, grid, block, 0, s, g, m0);
        else if (nm == 3) hipLaunchKernelGGL(k_gemv_bf16<3>, grid, block, 0, s, g, m0);
        else if (nm == 2) hipLaunchKernelGGL(k_gemv_bf16<2>, grid, block, 0, s, g, m0);
        else hipLaunchKernelGGL(k_gemv_bf16<1>, grid, block, 0, s, g, m0);
        if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
    }
    return hipSuccess;
}

} // namespace bl
