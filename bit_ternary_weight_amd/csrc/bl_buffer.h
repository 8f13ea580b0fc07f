// bl_buffer.h -- raw buffer resources for loads whose padding must move no
// data.  Internal to libbitlinear (the public ABI is include/bitlinear.h).
#pragma once

#include "bl_common.h"

namespace bl {

// Raw buffer resource over [p, p + bytes): a load at a byte offset past the
// range returns zeros without a memory access, so padding loads (issued only
// to keep a wave's load count fixed) cost no cache or memory traffic.  The
// last word is the data-format word of gfx9-family buffer resources.  p and
// bytes must be wave-uniform (the resource lives in scalar registers; the
// readfirstlane keeps the compiler from computing the size in vector
// registers, which would make it loop over the lanes around every load).
constexpr unsigned kBufOob = 0x80000000u;   // an offset past every range used here
constexpr int kBufNt = 2;                   // cache-policy operand: non-temporal
__device__ __forceinline__ __amdgpu_buffer_rsrc_t buf_rsrc(const void *p, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void *>(p), (short)0, __builtin_amdgcn_readfirstlane(bytes),
                                             0x00020000);
}
template <int AUX>
__device__ __forceinline__ v4i buf_ld16(__amdgpu_buffer_rsrc_t r, unsigned off) {
    return __builtin_amdgcn_raw_buffer_load_b128(r, (int)off, 0, AUX);
}

} // namespace bl
