// Peak probes for the benchmark (libpkm_probe.so): what this GPU sustains for
// a plain streaming read from HBM and for back-to-back bf16 MFMAs, measured in
// the same run as the kernels they are compared with.  Not part of the lookup
// and not in libpkm.so.
//
//   pkm_probe_stream_read: every 16-byte vector of src read once (non-temporal
//     loads, four in flight per lane, grid-stride over a chip-filling grid).
//   pkm_probe_mfma_bf16: each wave issues iters x 8 independent
//     v_mfma_f32_16x16x32_bf16 (16,384 flops each) or, with shape 1,
//     v_mfma_f32_32x32x16_bf16 (32,768 flops each) on register operands.
// Both fold their data into a value that is stored only when it equals a
// runtime key, so the loads and MFMAs cannot be removed.
#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include "common.h"

using namespace pkm;

namespace {

__global__ __launch_bounds__(256) void stream_read_kernel(const u32x4* __restrict__ src, int64_t nvec, uint32_t key,
                                                          uint32_t* __restrict__ out) {
  const int64_t stride = int64_t(gridDim.x) * 256;
  int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < nvec; i += 4 * stride) {
    const u32x4 a = ld16_nt(src + i);
    const u32x4 b = ld16_nt(src + i + stride);
    const u32x4 c = ld16_nt(src + i + 2 * stride);
    const u32x4 d = ld16_nt(src + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < nvec; i += stride) {
    const u32x4 a = ld16_nt(src + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == key) out[0] = acc;
}

typedef __attribute__((ext_vector_type(8))) __bf16 bf16x8_t;

__global__ __launch_bounds__(256) void mfma_loop_kernel(int iters, uint32_t key, uint32_t* __restrict__ out) {
  const uint32_t t = threadIdx.x * 2654435761u + blockIdx.x;
  const u32x4 av = {t & 0x3F803F80u, (t >> 3) & 0x3F803F80u, 0x3F003F00u, 0x3E803E80u};
  const u32x4 bv = {(t >> 5) & 0x3F803F80u, 0x3F003F00u, (t >> 7) & 0x3F803F80u, 0x3E803E80u};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
  f32x4 c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j) c[j] = f32x4{0.f, 0.f, 0.f, 0.f};
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j) s += c[j][0] + c[j][1] + c[j][2] + c[j][3];
  if (__float_as_uint(s) == key) out[0] = __float_as_uint(s);
}

typedef __attribute__((ext_vector_type(16))) float f32x16_t;

__global__ __launch_bounds__(256) void mfma32_loop_kernel(int iters, uint32_t key, uint32_t* __restrict__ out) {
  const uint32_t t = threadIdx.x * 2654435761u + blockIdx.x;
  const u32x4 av = {t & 0x3F803F80u, (t >> 3) & 0x3F803F80u, 0x3F003F00u, 0x3E803E80u};
  const u32x4 bv = {(t >> 5) & 0x3F803F80u, 0x3F003F00u, (t >> 7) & 0x3F803F80u, 0x3E803E80u};
  const bf16x8_t a = __builtin_bit_cast(bf16x8_t, av);
  const bf16x8_t b = __builtin_bit_cast(bf16x8_t, bv);
  f32x16_t c[8];
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) c[j][e] = 0.f;
  for (int it = 0; it < iters; ++it) {
#pragma unroll
    for (int j = 0; j < 8; ++j) c[j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(a, b, c[j], 0, 0, 0);
  }
  float s = 0.f;
#pragma unroll
  for (int j = 0; j < 8; ++j)
#pragma unroll
    for (int e = 0; e < 16; ++e) s += c[j][e];
  if (__float_as_uint(s) == key) out[0] = __float_as_uint(s);
}

}  // namespace

extern "C" {

// Reads bytes (a multiple of 16) from device memory src once.  out: one
// device uint32 (written only in the improbable case that the folded value
// equals key).  Returns 0 or a hipError_t.
int pkm_probe_stream_read(void* stream, const void* src, size_t bytes, int blocks, uint32_t key, uint32_t* out) {
  if (src == nullptr || out == nullptr || bytes % 16 || blocks < 1) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(stream_read_kernel, dim3(unsigned(blocks)), dim3(256), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u32x4*>(src), int64_t(bytes / 16), key, out);
  return int(hipGetLastError());
}

// blocks x 4 waves, each iters x 8 MFMAs: shape 0 16x16x32 bf16 (16,384 flops
// each), shape 1 32x32x16 bf16 (32,768 flops each).
int pkm_probe_mfma_bf16(void* stream, int blocks, int iters, int shape, uint32_t key, uint32_t* out) {
  if (out == nullptr || blocks < 1 || iters < 1 || shape < 0 || shape > 1) return int(hipErrorInvalidValue);
  hipLaunchKernelGGL(shape ? mfma32_loop_kernel : mfma_loop_kernel, dim3(unsigned(blocks)), dim3(256), 0,
                     static_cast<hipStream_t>(stream), iters, key, out);
  return int(hipGetLastError());
}

}  // extern "C"
