// bl_ste.h -- internal declarations of the training backward launches
// (k_ste.hip), used by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

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
                                 const float *w_mean, float *dX, void *ws, hipStream_t s);
// dW [N][K] = sum_m bf16(fp32(dY[m][n] / a[m])) * q[m][k]; dY bf16 or fp32.
hipError_t launch_ste_grad_weight(const void *dY, bool dy_bf16, int M, int N, int K, const int8_t *q, const float *a,
                                  float *dW, void *ws, hipStream_t s);

} // namespace bl
