// k_ste.hip -- the backward pass of BitLinear in quantization-aware training
// (the straight-through estimator): gradients pass through the weight and
// activation quantizers unchanged, so
//   dX = dY . W~          W~ = codes * w_mean, the fake-quantized weight
//   dW = dY^T . x~        x~ = q / a, the fake-quantized activations
// Article "Transformers 实战 BitNet 1.58 位量化", "BitLinear 的三步量化" (the
// QAT weight and activation quantizers, both with a straight-through
// backward that returns the incoming gradient unchanged).
//
// Both products run as one bf16 MFMA GEMM, C[i][j] = s * sum_l A[i][l] B[j][l]
// with both operands contiguous along l, after preparation launches that
// write the operands in bf16, zero-padded to whole tiles (rows to 128, the
// contraction to 64):
//   dX: A = dY [M][N] (used in place when it is bf16 and already whole tiles,
//       else rounded / copied), B = codes transposed [K][N] (exact), s = w_mean;
//   dW: A = bf16(fp32(dY[m][n] / a[m])) transposed [N][M], B = q transposed
//       [K][M] (exact), s = 1.
// The output gradient may be bf16 or fp32; an fp32 one is rounded to nearest
// even here (for dW after the division by a, one rounding).
// The GEMM: 128 x 128 output tiles, 4 waves of 64 x 64, 64-deep stages
// through LDS (pieces of a row permuted, the next stage's loads in flight in
// registers), v_mfma_f32_16x16x32_bf16 with the B fragment as the first
// operand so each lane ends with four consecutive outputs of one row
// (16-byte stores).
#include "bl_common.h"
#include "bl_ste.h"

namespace bl {

namespace {

typedef __bf16 bf16x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));

constexpr int kT = 128;            // output tile (both dimensions)
constexpr int kL = 64;             // contraction depth per stage
// LDS rows of 64 bf16 (128 bytes, 8 pieces of 16), unpadded: piece p of row r
// sits at position p ^ ((r >> 1) & 7).  Lane group g of a k-step ks reads
// piece (g & 1) | (g >> 1) << 2 | ks << 1 (a permutation of the k order that
// the two operands share), so the 16 lanes of a group, and lanes 0-7 with
// 32-39, touch distinct banks.
__device__ __forceinline__ int lds_pos(int r, int p) { return r * kL + 8 * (p ^ ((r >> 1) & 7)); }
__device__ __forceinline__ int k_piece(int g, int ks) { return (g & 1) | ((g >> 1) << 2) | (ks << 1); }

__device__ __forceinline__ __bf16 to_bf(float x) { return static_cast<__bf16>(x); }

// Codes of a plane-order packed weight, transposed and zero-padded:
// ct[k][n] = code(n, k) in bf16 (-1, 0, 1) for k < K, n < N = 4R, and 0 for
// K <= k < J or N <= n < L (ct is [J][L]).  Block: 32 packed rows x 64
// columns; thread (k = t >> 2, field f = t & 3) writes the rows n = f*R + r
// of its 32 packed rows r that exist.  The first column of blocks also
// clears the padding columns N .. L-1 of its 64 rows.
__global__ __launch_bounds__(256) void k_codes_t(const uint8_t *P, int R, int K, int L, __bf16 *ct) {
    __shared__ uint8_t tile[32][64 + 4];
    const int r0 = blockIdx.x * 32, k0 = blockIdx.y * 64, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = t + 256 * i, r = e >> 6, k = e & 63;
        tile[r][k] = (r0 + r < R && k0 + k < K) ? P[(size_t)(r0 + r) * K + k0 + k] : (uint8_t)0x55;
    }
    __syncthreads();
    const int k = t >> 2, f = t & 3;
    const bool krow = k0 + k < K;
    __bf16 *dst = ct + (size_t)(k0 + k) * L + f * R + r0;
    const bool vec = (R & 7) == 0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j)
            v[j] = to_bf(krow ? (float)(((tile[8 * c + j][k] >> (2 * f)) & 3) - 1) : 0.0f);
        if (vec && r0 + 8 * c + 8 <= R) {
            *reinterpret_cast<bf16x8 *>(dst + 8 * c) = v;
        } else {
#pragma unroll
            for (int j = 0; j < 8; ++j)
                if (r0 + 8 * c + j < R) dst[8 * c + j] = v[j];
        }
    }
    if (blockIdx.x == 0) {
        __bf16 *row = ct + (size_t)(k0 + k) * L;
        for (int n = 4 * R + f; n < L; n += 4) row[n] = to_bf(0.0f);
    }
}

// dst[i][l] = bf16(src[i][l]) for i < rows, l < cols, 0 elsewhere in the
// padded [I][L] destination (L a multiple of 8); 8 columns per thread.
template <typename T>
__global__ __launch_bounds__(256) void k_pad_bf16(const T *src, int rows, int cols, __bf16 *dst, int I, int L) {
    const size_t e = (size_t)blockIdx.x * 256 + threadIdx.x;
    const int per_row = L / 8;
    if (e >= (size_t)I * per_row) return;
    const int i = (int)(e / per_row), l0 = (int)(e % per_row) * 8;
    bf16x8 v;
#pragma unroll
    for (int j = 0; j < 8; ++j)
        v[j] = to_bf((i < rows && l0 + j < cols) ? (float)src[(size_t)i * cols + l0 + j] : 0.0f);
    *reinterpret_cast<bf16x8 *>(dst + (size_t)i * L + l0) = v;
}

// dst[c][r] = bf16(src[r][c] / a[r]) (SCALE) or bf16(src[r][c]) for a
// [rows][cols] source, zero outside it; dst is [C][R] with C, R multiples of
// 64 covering cols, rows.  64 x 64 blocks through LDS.
template <typename T, bool SCALE>
__global__ __launch_bounds__(256) void k_transpose(const T *src, int rows, int cols, const float *a, __bf16 *dst,
                                                   int R) {
    __shared__ float tile[64][64 + 1];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = t + 256 * i, r = e >> 6, c = e & 63;
        float v = 0.0f;
        if (r0 + r < rows && c0 + c < cols) {
            v = (float)src[(size_t)(r0 + r) * cols + c0 + c];
            if (SCALE) v = v / a[r0 + r];
        }
        tile[r][c] = v;
    }
    __syncthreads();
    const int c = t >> 2, q = (t & 3) * 16;
    __bf16 *d = dst + (size_t)(c0 + c) * R + r0 + q;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = to_bf(tile[q + 8 * h + j][c]);
        *reinterpret_cast<bf16x8 *>(d + 8 * h) = v;
    }
}

__device__ __forceinline__ f32x4 mfma_bf16(bf16x8 a, bf16x8 b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c, 0, 0, 0);
}

// C[i][j] = epilogue(sum_l A[i][l] B[j][l]) for i < Ir, j < Jr; A [I][L],
// B [J][L] bf16 (zero-padded), C [Ir][Jr] with row stride Jr; I, J, L
// multiples of 128, 128, 64.  Epilogues:
//   EPI_SCALE: C = s * sum, s read from device memory (1 if null), fp32 or
//     (e.y_dt = BL_BF16) rounded to bf16;
//   EPI_BITLINEAR: the BitLinear rescale of an exact integer sum (the
//     operands are int8 activation codes and ternary codes, every partial sum
//     an integer below 2^24, so the fp32 accumulator holds it exactly):
//     C = float(sum) * (w_mean[seg(j)] / a[i]) in fp32, its bf16 rounding, or
//     the int32 sum itself, per e.y_dt.
constexpr int EPI_SCALE = 0;
constexpr int EPI_BITLINEAR = 1;

template <int EPI>
__global__ __launch_bounds__(256) void k_gemm_nt_bf16(const __bf16 *A, const __bf16 *B, void *Cv, int I, int J,
                                                       int L, int Ir, int Jr, const float *s_ptr, GemmEpi e) {
    float *C = static_cast<float *>(Cv);
    const float s = (EPI == EPI_SCALE && s_ptr) ? *s_ptr : 1.0f;
    __shared__ __attribute__((aligned(16))) __bf16 as[kT * kL];
    __shared__ __attribute__((aligned(16))) __bf16 bs[kT * kL];
    const int nj = J / kT;
    const int i0 = (int)(blockIdx.x / nj) * kT, j0 = (int)(blockIdx.x % nj) * kT;
    const int t = threadIdx.x, w = t >> 6, lane = t & 63, g = lane >> 4, lr = lane & 15;
    const int wi = (w >> 1) * 64, wj = (w & 1) * 64;
    // staging: 1024 16-byte pieces per operand tile (row e >> 3, piece e & 7), 4 per thread
    bf16x8 ar[4], br[4];
    auto fetch = [&](int l0) {
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = t + 256 * r;
            ar[r] = *reinterpret_cast<const bf16x8 *>(A + (size_t)(i0 + (e >> 3)) * L + l0 + 8 * (e & 7));
            br[r] = *reinterpret_cast<const bf16x8 *>(B + (size_t)(j0 + (e >> 3)) * L + l0 + 8 * (e & 7));
        }
    };
    f32x4 acc[4][4];
#pragma unroll
    for (int x = 0; x < 4; ++x)
#pragma unroll
        for (int y = 0; y < 4; ++y) acc[x][y] = f32x4{0.0f, 0.0f, 0.0f, 0.0f};
    const int nst = L / kL;
    fetch(0);
    for (int st = 0; st < nst; ++st) {
        __syncthreads();
#pragma unroll
        for (int r = 0; r < 4; ++r) {
            const int e = t + 256 * r;
            *reinterpret_cast<bf16x8 *>(&as[lds_pos(e >> 3, e & 7)]) = ar[r];
            *reinterpret_cast<bf16x8 *>(&bs[lds_pos(e >> 3, e & 7)]) = br[r];
        }
        __syncthreads();
        if (st + 1 < nst) fetch((st + 1) * kL);
        // raised wave priority over the stage's products: the two
        // workgroups of a CU then take turns at the matrix cores instead of
        // meeting at the same barrier (6-10 % on the backward GEMMs)
        __builtin_amdgcn_s_setprio(1);
#pragma unroll
        for (int ks = 0; ks < kL / 32; ++ks) {
            bf16x8 af[4], bf[4];
#pragma unroll
            for (int x = 0; x < 4; ++x)
                af[x] = *reinterpret_cast<const bf16x8 *>(&as[lds_pos(wi + 16 * x + lr, k_piece(g, ks))]);
#pragma unroll
            for (int y = 0; y < 4; ++y)
                bf[y] = *reinterpret_cast<const bf16x8 *>(&bs[lds_pos(wj + 16 * y + lr, k_piece(g, ks))]);
            // B first: lane (g, lr) accumulates C[i = 16x + lr][j = 16y + 4g + 0..3]
#pragma unroll
            for (int x = 0; x < 4; ++x)
#pragma unroll
                for (int y = 0; y < 4; ++y) acc[x][y] = mfma_bf16(bf[y], af[x], acc[x][y]);
        }
        __builtin_amdgcn_s_setprio(0);
    }
    const bool whole = i0 + kT <= Ir && j0 + kT <= Jr && (Jr & 3) == 0;
    if constexpr (EPI == EPI_BITLINEAR) {
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = i0 + wi + 16 * x + lr;
            const float ai = i < Ir ? e.a[i] : 1.0f;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                const int j = j0 + wj + 4 * g + 16 * y;
                float v[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) {
                    int sg = 0;
#pragma unroll
                    for (int t = 0; t < BL_MAX_SEGMENTS - 1; ++t)
                        sg += (t + 1 < e.nseg && j + c >= e.cend[t]) ? 1 : 0;
                    v[c] = acc[x][y][c] * (e.w_mean[sg] / ai);
                }
                const size_t o = (size_t)i * Jr + j;
                if (e.y_dt == BL_I32) {
                    int *Ci = static_cast<int *>(Cv);
                    if (whole) {
                        *reinterpret_cast<int4 *>(Ci + o) =
                            int4{(int)acc[x][y][0], (int)acc[x][y][1], (int)acc[x][y][2], (int)acc[x][y][3]};
                    } else if (i < Ir) {
                        for (int c = 0; c < 4; ++c)
                            if (j + c < Jr) Ci[o + c] = (int)acc[x][y][c];
                    }
                } else if (e.y_dt == BL_BF16) {
                    uint16_t *Cb = static_cast<uint16_t *>(Cv);
                    if (whole) {
                        uint2 pk;
                        pk.x = (uint32_t)f32_to_bf16(v[0]) | ((uint32_t)f32_to_bf16(v[1]) << 16);
                        pk.y = (uint32_t)f32_to_bf16(v[2]) | ((uint32_t)f32_to_bf16(v[3]) << 16);
                        *reinterpret_cast<uint2 *>(Cb + o) = pk;
                    } else if (i < Ir) {
                        for (int c = 0; c < 4; ++c)
                            if (j + c < Jr) Cb[o + c] = f32_to_bf16(v[c]);
                    }
                } else {
                    if (whole) {
                        *reinterpret_cast<float4 *>(C + o) = float4{v[0], v[1], v[2], v[3]};
                    } else if (i < Ir) {
                        for (int c = 0; c < 4; ++c)
                            if (j + c < Jr) C[o + c] = v[c];
                    }
                }
            }
        }
        return;
    }
    if (e.y_dt == BL_BF16) {
        // the scaled sums rounded to bf16 (round to nearest even), the
        // caller's compute type
        uint16_t *Cb = static_cast<uint16_t *>(Cv);
#pragma unroll
        for (int x = 0; x < 4; ++x) {
            const int i = i0 + wi + 16 * x + lr;
            uint16_t *crow = Cb + (size_t)i * Jr + j0 + wj + 4 * g;
#pragma unroll
            for (int y = 0; y < 4; ++y) {
                uint16_t h[4];
#pragma unroll
                for (int c = 0; c < 4; ++c) h[c] = f32_to_bf16(acc[x][y][c] * s);
                if (whole) {
                    *reinterpret_cast<uint2 *>(crow + 16 * y) =
                        make_uint2((uint32_t)h[0] | ((uint32_t)h[1] << 16), (uint32_t)h[2] | ((uint32_t)h[3] << 16));
                } else if (i < Ir) {
                    const int j = j0 + wj + 4 * g + 16 * y;
#pragma unroll
                    for (int c = 0; c < 4; ++c)
                        if (j + c < Jr) crow[16 * y + c] = h[c];
                }
            }
        }
        return;
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        const int i = i0 + wi + 16 * x + lr;
        float *crow = C + (size_t)i * Jr + j0 + wj + 4 * g;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            float4 v;
            v.x = acc[x][y][0] * s;
            v.y = acc[x][y][1] * s;
            v.z = acc[x][y][2] * s;
            v.w = acc[x][y][3] * s;
            if (whole) {
                *reinterpret_cast<float4 *>(crow + 16 * y) = v;
            } else if (i < Ir) {
                const int j = j0 + wj + 4 * g + 16 * y;
                if (j + 0 < Jr) crow[16 * y + 0] = v.x;
                if (j + 1 < Jr) crow[16 * y + 1] = v.y;
                if (j + 2 < Jr) crow[16 * y + 2] = v.z;
                if (j + 3 < Jr) crow[16 * y + 3] = v.w;
            }
        }
    }
}

inline int pad_to(int x, int m) { return (x + m - 1) / m * m; }

// dX operand A is taken in place when it is already bf16 in whole tiles.
bool dy_in_place(int M, int N, bool dy_bf16) { return dy_bf16 && M % kT == 0 && N % kL == 0; }

} // namespace

size_t ste_grad_input_ws_bytes(int M, int N, int K, bool dy_bf16) {
    const size_t L = pad_to(N, kL), I = pad_to(M, kT), J = pad_to(K, kT);
    const size_t ct = (J * L * sizeof(__bf16) + 255) & ~(size_t)255;
    return ct + (dy_in_place(M, N, dy_bf16) ? 0 : I * L * sizeof(__bf16));
}

size_t ste_grad_weight_ws_bytes(int M, int N, int K) {
    const size_t L = pad_to(M, kL), I = pad_to(N, kT), J = pad_to(K, kT);
    return ((I * L * sizeof(__bf16) + 255) & ~(size_t)255) + J * L * sizeof(__bf16);
}

bool ste_dims_fit(int M, int N, int K) {
    const size_t a = pad_to(M, kT), b = pad_to(N, kT), c = pad_to(K, kT);
    const size_t lim = (size_t)1 << 31;
    return a * b < lim && a * c < lim && b * c < lim;
}

hipError_t launch_ste_grad_input(const void *dY, bool dy_bf16, int M, int N, int K, const uint8_t *packed,
                                 const float *w_mean, void *dX, bool dx_bf16, void *ws, hipStream_t s) {
    const int L = pad_to(N, kL), I = pad_to(M, kT), J = pad_to(K, kT), R = N / 4;
    __bf16 *ct = static_cast<__bf16 *>(ws);
    hipLaunchKernelGGL(k_codes_t, dim3((R + 31) / 32, J / 64), dim3(256), 0, s, packed, R, K, L, ct);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    const __bf16 *A = static_cast<const __bf16 *>(dY);
    if (!dy_in_place(M, N, dy_bf16)) {
        __bf16 *dyb = reinterpret_cast<__bf16 *>(static_cast<char *>(ws) +
                                                 (((size_t)J * L * sizeof(__bf16) + 255) & ~(size_t)255));
        const size_t threads = (size_t)I * (L / 8);
        const dim3 grid((unsigned)((threads + 255) / 256));
        if (dy_bf16)
            hipLaunchKernelGGL(k_pad_bf16<__bf16>, grid, dim3(256), 0, s, static_cast<const __bf16 *>(dY), M, N, dyb,
                               I, L);
        else
            hipLaunchKernelGGL(k_pad_bf16<float>, grid, dim3(256), 0, s, static_cast<const float *>(dY), M, N, dyb, I,
                               L);
        if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
        A = dyb;
    }
    GemmEpi e{};
    e.y_dt = dx_bf16 ? BL_BF16 : BL_F32;
    hipLaunchKernelGGL(k_gemm_nt_bf16<EPI_SCALE>, dim3((I / kT) * (J / kT)), dim3(256), 0, s, A, ct, dX, I, J, L, M,
                       K, w_mean, e);
    return hipGetLastError();
}

hipError_t launch_ste_grad_weight(const void *dY, bool dy_bf16, int M, int N, int K, const int8_t *q, const float *a,
                                  float *dW, void *ws, hipStream_t s) {
    const int L = pad_to(M, kL), I = pad_to(N, kT), J = pad_to(K, kT);
    __bf16 *at = static_cast<__bf16 *>(ws);                                        // [I][L]
    __bf16 *qt = reinterpret_cast<__bf16 *>(static_cast<char *>(ws) +
                                            (((size_t)I * L * sizeof(__bf16) + 255) & ~(size_t)255));  // [J][L]
    if (dy_bf16)
        hipLaunchKernelGGL((k_transpose<__bf16, true>), dim3(I / 64, L / 64), dim3(256), 0, s,
                           static_cast<const __bf16 *>(dY), M, N, a, at, L);
    else
        hipLaunchKernelGGL((k_transpose<float, true>), dim3(I / 64, L / 64), dim3(256), 0, s,
                           static_cast<const float *>(dY), M, N, a, at, L);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((k_transpose<int8_t, false>), dim3(J / 64, L / 64), dim3(256), 0, s, q, M, K, nullptr, qt, L);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemm_nt_bf16<EPI_SCALE>, dim3((I / kT) * (J / kT)), dim3(256), 0, s, at, qt, (void *)dW, I, J,
                       L, N, K, nullptr, GemmEpi{});
    return hipGetLastError();
}

size_t unpacked_gemm_ws_bytes(int M, int K) { return (size_t)pad_to(M, kT) * K * sizeof(__bf16); }

bool unpacked_gemm_fits(int M, int N, int K) {
    return K % kL == 0 && N % kT == 0 && (size_t)pad_to(M, kT) * K < ((size_t)1 << 31) &&
           (size_t)N * K < ((size_t)1 << 31) && (size_t)pad_to(M, kT) * N < ((size_t)1 << 31);
}

hipError_t launch_unpacked_gemm(const int8_t *q, const float *a, int M, int K, const __bf16 *W, int N,
                                const GemmEpi &e, void *y, void *ws, hipStream_t s) {
    const int I = pad_to(M, kT);
    __bf16 *qb = static_cast<__bf16 *>(ws);   // [I][K] bf16 codes, zero rows below M
    const size_t threads = (size_t)I * (K / 8);
    hipLaunchKernelGGL(k_pad_bf16<int8_t>, dim3((unsigned)((threads + 255) / 256)), dim3(256), 0, s, q, M, K, qb, I, K);
    if (hipError_t err = hipGetLastError(); err != hipSuccess) return err;
    GemmEpi ep = e;
    ep.a = a;
    hipLaunchKernelGGL(k_gemm_nt_bf16<EPI_BITLINEAR>, dim3((I / kT) * (N / kT)), dim3(256), 0, s, qb, W, y, I, N, K,
                       M, N, nullptr, ep);
    return hipGetLastError();
}

} // namespace bl
