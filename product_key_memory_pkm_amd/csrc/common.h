// Device helpers shared by the PKM kernels (gfx950, wave64).
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace pkm {

constexpr int kWave = 64;

typedef __attribute__((ext_vector_type(4))) float f32x4;
typedef __attribute__((ext_vector_type(16))) float f32x16;
typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8;
typedef __attribute__((ext_vector_type(2))) __bf16 bf16x2;
typedef __attribute__((ext_vector_type(4))) uint32_t u32x4;
typedef __attribute__((ext_vector_type(2))) uint32_t u32x2;

// Storage element types.  bf16 is carried as raw 16-bit patterns.
struct bf16_t {
  uint16_t bits;
};

__device__ __forceinline__ float bf16_to_f32(uint16_t b) { return __uint_as_float(uint32_t(b) << 16); }

// Round-to-nearest-even fp32 -> bf16 (finite inputs).
__device__ __forceinline__ uint16_t f32_to_bf16(float f) {
  uint32_t u = __float_as_uint(f);
  u += 0x7FFFu + ((u >> 16) & 1u);
  return uint16_t(u >> 16);
}

// Low / high bf16 of a packed 32-bit word, widened to fp32.
__device__ __forceinline__ float bf16lo(uint32_t w) { return __uint_as_float(w << 16); }
__device__ __forceinline__ float bf16hi(uint32_t w) { return __uint_as_float(w & 0xFFFF0000u); }

__device__ __forceinline__ uint32_t pack_bf16x2(float lo, float hi) {
  return uint32_t(f32_to_bf16(lo)) | (uint32_t(f32_to_bf16(hi)) << 16);
}

// Order-preserving map of a finite fp32 onto uint32 (larger float -> larger key).
// -0.0 is first turned into +0.0 so the two compare equal.  Every finite value
// maps to a key >= 0x007FFFFF, so 0 can mark an empty slot.
__device__ __forceinline__ uint32_t float_key(float f) {
  uint32_t u = __float_as_uint(f + 0.0f);
  return (u & 0x80000000u) ? ~u : (u | 0x80000000u);
}
__device__ __forceinline__ float key_float(uint32_t k) {
  uint32_t u = (k & 0x80000000u) ? (k & 0x7FFFFFFFu) : ~k;
  return __uint_as_float(u);
}

__device__ __forceinline__ int lane_id() { return __lane_id(); }

__device__ __forceinline__ uint64_t ballot(bool p) { return __ballot(p); }
__device__ __forceinline__ int popc64(uint64_t m) { return __popcll(m); }

__device__ __forceinline__ uint32_t shfl_xor_u32(uint32_t v, int m) {
  return (uint32_t)__shfl_xor((int)v, m, kWave);
}
__device__ __forceinline__ uint64_t shfl_xor_u64(uint64_t v, int m) {
  uint32_t lo = shfl_xor_u32(uint32_t(v), m);
  uint32_t hi = shfl_xor_u32(uint32_t(v >> 32), m);
  return (uint64_t(hi) << 32) | lo;
}
__device__ __forceinline__ float shfl_f32(float v, int src) { return __shfl(v, src, kWave); }
__device__ __forceinline__ int shfl_i32(int v, int src) { return __shfl(v, src, kWave); }

__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}
// Sum over the 64 lanes with DPP moves only (no LDS traffic): quad, half-row,
// row, then across the four rows; the total lands in lane 63 and is broadcast.
__device__ __forceinline__ float wave_sum_dpp(float v) {
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0xB1, 0xF, 0xF, false));   // quad_perm 1,0,3,2
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x4E, 0xF, 0xF, false));   // quad_perm 2,3,0,1
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x141, 0xF, 0xF, false));  // row_half_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x140, 0xF, 0xF, false));  // row_mirror
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x142, 0xA, 0xF, false));  // row_bcast:15
  v += __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(v), 0x143, 0xC, 0xF, false));  // row_bcast:31
  return __int_as_float(__builtin_amdgcn_readlane(__float_as_int(v), 63));
}

__device__ __forceinline__ float wave_max(float v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v = fmaxf(v, __shfl_xor(v, m, kWave));
  return v;
}
__device__ __forceinline__ int wave_sum_i(int v) {
#pragma unroll
  for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, kWave);
  return v;
}

// Exclusive prefix sum of one int per lane across the wave.
__device__ __forceinline__ int wave_excl_scan(int v, int* total) {
  int lane = lane_id();
  int x = v;
#pragma unroll
  for (int d = 1; d < kWave; d <<= 1) {
    int y = __shfl_up(x, d, kWave);
    if (lane >= d) x += y;
  }
  *total = __shfl(x, kWave - 1, kWave);
  return x - v;
}

// k-th largest (1 <= k <= number of lanes holding real values) of one uint32 per
// lane, by bisection on the bits: the largest T with #{lanes: v >= T} >= k.
__device__ __forceinline__ uint32_t wave_kth_largest_u32(uint32_t v, int k) {
  uint32_t res = 0;
#pragma unroll
  for (int b = 31; b >= 0; --b) {
    uint32_t cand = res | (1u << b);
    if (popc64(ballot(v >= cand)) >= k) res = cand;
  }
  return res;
}

// Bitonic sort of one uint64 per lane across the wave, descending (lane 0 largest).
__device__ __forceinline__ uint64_t wave_sort_desc_u64(uint64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= kWave; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      uint64_t o = shfl_xor_u64(v, stride);
      bool lower = (lane & stride) == 0;
      bool desc = (lane & size) == 0;
      bool take_max = (lower == desc);
      uint64_t mx = v > o ? v : o;
      uint64_t mn = v > o ? o : v;
      v = take_max ? mx : mn;
    }
  }
  return v;
}

// Round an fp32 value to the storage type.
template <typename T>
__device__ __forceinline__ T to_storage(float v);
template <>
__device__ __forceinline__ float to_storage<float>(float v) { return v; }
template <>
__device__ __forceinline__ bf16_t to_storage<bf16_t>(float v) { return bf16_t{f32_to_bf16(v)}; }

template <typename T>
__device__ __forceinline__ float to_f32(T v);
template <>
__device__ __forceinline__ float to_f32<float>(float v) { return v; }
template <>
__device__ __forceinline__ float to_f32<bf16_t>(bf16_t v) { return bf16_to_f32(v.bits); }

// 16 bytes of storage elements widened to fp32: 8 bf16 or 4 fp32.
template <typename T>
struct Vec16;
template <>
struct Vec16<bf16_t> {
  static constexpr int N = 8;
  __device__ __forceinline__ static void widen(const u32x4& r, float* f) {
    f[0] = bf16lo(r.x); f[1] = bf16hi(r.x); f[2] = bf16lo(r.y); f[3] = bf16hi(r.y);
    f[4] = bf16lo(r.z); f[5] = bf16hi(r.z); f[6] = bf16lo(r.w); f[7] = bf16hi(r.w);
  }
  __device__ __forceinline__ static u32x4 narrow(const float* f) {
    u32x4 r;
    r.x = pack_bf16x2(f[0], f[1]); r.y = pack_bf16x2(f[2], f[3]);
    r.z = pack_bf16x2(f[4], f[5]); r.w = pack_bf16x2(f[6], f[7]);
    return r;
  }
};
template <>
struct Vec16<float> {
  static constexpr int N = 4;
  __device__ __forceinline__ static void widen(const u32x4& r, float* f) {
    f[0] = __uint_as_float(r.x); f[1] = __uint_as_float(r.y);
    f[2] = __uint_as_float(r.z); f[3] = __uint_as_float(r.w);
  }
  __device__ __forceinline__ static u32x4 narrow(const float* f) {
    u32x4 r;
    r.x = __float_as_uint(f[0]); r.y = __float_as_uint(f[1]);
    r.z = __float_as_uint(f[2]); r.w = __float_as_uint(f[3]);
    return r;
  }
};

__device__ __forceinline__ u32x4 ld16(const void* p) { return *reinterpret_cast<const u32x4*>(p); }
__device__ __forceinline__ u32x4 ld16_nt(const void* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const u32x4*>(p));
}
__device__ __forceinline__ void st16(void* p, const u32x4& v) { *reinterpret_cast<u32x4*>(p) = v; }

}  // namespace pkm
