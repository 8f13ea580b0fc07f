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
// with both operands contiguous along l, after a preparation launch:
//   dX: A = dY [M][N] as given (bf16), B = codes transposed [K][N] (bf16,
//       exact), s = w_mean;
//   dW: A = bf16(dY[m][n] / a[m]) transposed [N][M], B = q transposed [K][M]
//       (bf16, exact), s = 1.
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

// Codes of a plane-order packed weight, transposed: ct[k][n] = code(n, k) in
// bf16 (-1, 0, 1).  Block: 32 packed rows x 64 columns; thread (k = t >> 2,
// field f = t & 3) writes the 32 consecutive rows n = f*R + r0 .. +31.
__global__ __launch_bounds__(256) void k_codes_t(const uint8_t *P, int R, int K, __bf16 *ct) {
    __shared__ uint8_t tile[32][64 + 4];
    const int r0 = blockIdx.x * 32, k0 = blockIdx.y * 64, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int e = t + 256 * i, r = e >> 6, k = e & 63;
        tile[r][k] = P[(size_t)(r0 + r) * K + k0 + k];
    }
    __syncthreads();
    const int k = t >> 2, f = t & 3;
    __bf16 *dst = ct + (size_t)(k0 + k) * (4 * R) + f * R + r0;
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        bf16x8 v;
#pragma unroll
        for (int j = 0; j < 8; ++j) v[j] = to_bf((float)(((tile[8 * c + j][k] >> (2 * f)) & 3) - 1));
        *reinterpret_cast<bf16x8 *>(dst + 8 * c) = v;
    }
}

// dst[c][r] = bf16(src[r][c] / a[r]) (bf16 src, SCALE) or bf16(src[r][c])
// (int8 src) for a [rows][cols] source; 64 x 64 blocks through LDS.
template <typename T, bool SCALE>
__global__ __launch_bounds__(256) void k_transpose(const T *src, int rows, int cols, const float *a, __bf16 *dst) {
    __shared__ float tile[64][64 + 1];
    const int r0 = blockIdx.y * 64, c0 = blockIdx.x * 64, t = threadIdx.x;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int e = t + 256 * i, r = e >> 6, c = e & 63;
        float v = (float)src[(size_t)(r0 + r) * cols + c0 + c];
        if (SCALE) v = v / a[r0 + r];
        tile[r][c] = v;
    }
    __syncthreads();
    const int c = t >> 2, q = (t & 3) * 16;
    __bf16 *d = dst + (size_t)(c0 + c) * rows + r0 + q;
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

// C[i][j] = s * sum_l A[i][l] B[j][l]; A [I][L], B [J][L] bf16, C [I][J] fp32;
// I, J, L multiples of 128, 128, 64; s read from device memory (1 if null).
__global__ __launch_bounds__(256) void k_gemm_nt_bf16(const __bf16 *A, const __bf16 *B, float *C, int I, int J,
                                                       int L, const float *s_ptr) {
    const float s = s_ptr ? *s_ptr : 1.0f;
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
    }
#pragma unroll
    for (int x = 0; x < 4; ++x) {
        float *crow = C + (size_t)(i0 + wi + 16 * x + lr) * J + j0 + wj + 4 * g;
#pragma unroll
        for (int y = 0; y < 4; ++y) {
            float4 v;
            v.x = acc[x][y][0] * s;
            v.y = acc[x][y][1] * s;
            v.z = acc[x][y][2] * s;
            v.w = acc[x][y][3] * s;
            *reinterpret_cast<float4 *>(crow + 16 * y) = v;
        }
    }
}

} // namespace

size_t ste_grad_input_ws_bytes(int N, int K) { return (size_t)K * N * sizeof(__bf16); }
size_t ste_grad_weight_ws_bytes(int M, int N, int K) { return ((size_t)N * M + (size_t)K * M) * sizeof(__bf16); }

hipError_t launch_ste_grad_input(const __bf16 *dY, int M, int N, int K, const uint8_t *packed, const float *w_mean,
                                 float *dX, void *ws, hipStream_t s) {
    __bf16 *ct = static_cast<__bf16 *>(ws);
    const int R = N / 4;
    hipLaunchKernelGGL(k_codes_t, dim3(R / 32, K / 64), dim3(256), 0, s, packed, R, K, ct);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemm_nt_bf16, dim3((M / kT) * (K / kT)), dim3(256), 0, s, dY, ct, dX, M, K, N, w_mean);
    return hipGetLastError();
}

hipError_t launch_ste_grad_weight(const __bf16 *dY, int M, int N, int K, const int8_t *q, const float *a, float *dW,
                                  void *ws, hipStream_t s) {
    __bf16 *at = static_cast<__bf16 *>(ws);          // [N][M]
    __bf16 *qt = at + (size_t)N * M;                 // [K][M]
    hipLaunchKernelGGL((k_transpose<__bf16, true>), dim3(N / 64, M / 64), dim3(256), 0, s, dY, M, N, a, at);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL((k_transpose<int8_t, false>), dim3(K / 64, M / 64), dim3(256), 0, s, q, M, K, nullptr, qt);
    if (hipError_t e = hipGetLastError(); e != hipSuccess) return e;
    hipLaunchKernelGGL(k_gemm_nt_bf16, dim3((N / kT) * (K / kT)), dim3(256), 0, s, at, qt, dW, N, K, M, nullptr);
    return hipGetLastError();
}

} // namespace bl
