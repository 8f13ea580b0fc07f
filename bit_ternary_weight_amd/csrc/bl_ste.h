// bl_ste.h -- internal declarations of the training backward launches
// (k_ste.hip), used by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

namespace bl {

// Workspace bytes: the transposed codes (dX), the scaled transposed gradient
// and the transposed activation codes (dW), all bf16.
size_t ste_grad_input_ws_bytes(int N, int K);
size_t ste_grad_weight_ws_bytes(int M, int N, int K);
// dX [M][K] = (dY [M][N] . codes [N][K]) * w_mean[0] (device); M, N, K multiples of 128.
hipError_t launch_ste_grad_input(const __bf16 *dY, int M, int N, int K, const uint8_t *packed, const float *w_mean,
                                 float *dX, void *ws, hipStream_t s);
// dW [N][K] = sum_m bf16(dY[m][n] / a[m]) * q[m][k]; M, N, K multiples of 128.
hipError_t launch_ste_grad_weight(const __bf16 *dY, int M, int N, int K, const int8_t *q, const float *a, float *dW,
                                  void *ws, hipStream_t s);

} // namespace bl
