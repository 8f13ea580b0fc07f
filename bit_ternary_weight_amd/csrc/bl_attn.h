// bl_attn.h -- internal declarations of the prefill attention launches
// (k_attn_prefill.hip), used by the C ABI layer.
#pragma once
#include <hip/hip_runtime.h>
#include <stddef.h>

namespace bl {

// Workspace bytes of a prefill of M tokens: bf16 rotated queries and keys and
// the transposed bf16 values, each padded to a multiple of 64 tokens.
size_t attn_prefill_workspace_bytes(int M, int n_heads, int n_kv_heads);
// The two launches (RoPE / conversion / cache stores, then the attention).
hipError_t launch_attn_prefill(const float *q, const float *k, const float *v, int ldx, int M, int H, int KVH,
                               float *k_cache, float *v_cache, int max_seq, const float *rcos, const float *rsin,
                               float *out, int ldo, void *ws, hipStream_t s);

} // namespace bl
