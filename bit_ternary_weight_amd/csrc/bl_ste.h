// bl_ste.h -- internal declarations of the training backward launches
// (k_ste.hip), used by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "bitlinear.h"

namespace bl {

// Epilogue arguments of the bf16 GEMM when it computes a BitLinear product
// on unpacked codes: per-row activation scales a, per-segment weight scales,
// the exclusive end column of each segment, the output dtype.
struct GemmEpi {
    const float *a;
    const float *w_mean;
    int nseg;
    int cend[BL_MAX_SEGMENTS];
    int y_dt;
};

// Workspace bytes: the transposed codes and, unless the bf16 gradient is used
// in place, its padded bf16 copy (dX); the scaled transposed gradient and the
// transposed activation codes (dW); all bf16, padded to whole tiles.
size_t ste_grad_input_ws_bytes(int M, int N, int K, bool dy_bf16);
size_t ste_grad_weight_ws_bytes(int M, int N, int K);
// The padded operand and output sizes fit the kernels' 32-bit indexing.
bool ste_dims_fit(int M, int N, int K);
// dX [M][K] = (dY [M][N] . codes [N][K]) * w_mean[0] (device); dY bf16 or fp32
// (rounded to bf16); N a multiple of 4.
hipError_t launch_ste_grad_input(const void *dY, bool dy_bf16, int M, int N, int K, const uint8_t *packed,
                                 const float *w_mean, void *dX, bool dx_bf16, void *ws, hipStream_t s);
// dW [N][K] = sum_m bf16(fp32(dY[m][n] / a[m])) * q[m][k]; dY bf16 or fp32.
hipError_t launch_ste_grad_weight(const void *dY, bool dy_bf16, int M, int N, int K, const int8_t *q, const float *a,
                                  float *dW, void *ws, hipStream_t s);

// The offline-unpacked BitLinear product (bf16 codes): y [M][N] = rescale of
// q [M][K] (int8 codes, scales a) times W [N][K]^T (bf16 codes); needs
// unpacked_gemm_fits(M, N, K) and unpacked_gemm_ws_bytes(M, K) of scratch.
size_t unpacked_gemm_ws_bytes(int M, int K);
bool unpacked_gemm_fits(int M, int N, int K);
bool unpacked_gemv_fits(int K);
// Decode sizes: 4 token rows per pass, one wave per weight row (k_unpacked.hip).
hipError_t launch_unpacked_gemv(const int8_t *q, const float *a, int M, int K, const void *W, int N, const GemmEpi &e,
                                void *y, hipStream_t s);
hipError_t launch_unpacked_gemm(const int8_t *q, const float *a, int M, int K, const __bf16 *W, int N,
                                const GemmEpi &e, void *y, void *ws, hipStream_t s);

} // namespace bl
