// Cross-lane exchanges for the selection kernels (sorting networks): the value
// of lane (lane ^ stride) without going through LDS where the hardware allows.
#pragma once
#include "common.h"

namespace pkm {

// Value of lane (lane ^ stride): DPP quad permutes for strides 1 and 2,
// ds_swizzle (xor within 32 lanes, no address register) for 4..16, a
// bpermute for 32.  stride is a constant once the callers' loops unroll.
__device__ __forceinline__ uint32_t xor_lane(uint32_t v, int stride) {
  switch (stride) {
    case 1: return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0xB1, 0xF, 0xF, false));  // quad_perm 1,0,3,2
    case 2: return uint32_t(__builtin_amdgcn_update_dpp(0, int(v), 0x4E, 0xF, 0xF, false));  // quad_perm 2,3,0,1
    case 4: return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), (4 << 10) | 0x1F));
    case 8: return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), (8 << 10) | 0x1F));
    case 16: return uint32_t(__builtin_amdgcn_ds_swizzle(int(v), (16 << 10) | 0x1F));
    default: return uint32_t(__shfl_xor(int(v), stride, 64));
  }
}
__device__ __forceinline__ uint64_t xor_lane_u64(uint64_t v, int stride) {
  return (uint64_t(xor_lane(uint32_t(v >> 32), stride)) << 32) | xor_lane(uint32_t(v), stride);
}

}  // namespace pkm
