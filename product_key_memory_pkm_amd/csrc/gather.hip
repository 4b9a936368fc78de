// Step a6: softmax-weighted sum of value rows, heads summed (an embedding bag).
//
//   y[t, :] = sum_{h, s} w[t, h, s] * V[idx[t, h, s], :]
//
// Value matrix [K1*K2, d] read only at the selected rows, weights from the
// softmax over the selected keys ("Meta AI 可扩展内存层", sections 5.3 and 9.2;
// product-key paper summary, method details).
//
// Design (HBM bound: each selected row is a random d_value*elem-byte read):
//  * one wave per token and column block; the wave's 64 lanes split a row into
//    16-byte vectors, so a row read is contiguous across the wave;
//  * row indices and weights are loaded once per 64 rows (one per lane) and
//    broadcast with readlane, so row addresses are wave-uniform (SGPR base);
//  * U rows are issued back to back before any FMA, keeping U*NVL 16-byte
//    loads per lane in flight; V is read with non-temporal loads since random
//    rows of a multi-GB table are not reused through the caches;
//  * fp32 accumulation in registers, one rounding to the storage type.
#include "common.h"
#include "kernels.h"

namespace pkm {

template <typename T, int NVL, int U>
__global__ __launch_bounds__(256) void gather_sum_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const T* __restrict__ V, T* __restrict__ y,
                                                         int64_t ntok, int R, int nvec) {
  constexpr int E = Vec16<T>::N;  // elements per 16-byte vector
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const int v0 = blockIdx.y * (64 * NVL);
  const size_t row_bytes = size_t(nvec) * 16;
  const char* Vb = reinterpret_cast<const char*>(V);

  bool valid[NVL];
  int voff[NVL];
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    int v = v0 + m * 64 + lane;
    valid[m] = v < nvec;
    voff[m] = v * 16;
  }
  float acc[NVL][E];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[m][e] = 0.f;

  const int32_t* it = idx + t * R;
  const float* wt = w + t * R;
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int n = min(64, R - r0);
    const int my = r0 + lane;
    const int my_idx = my < R ? it[my] : 0;
    const float my_w = my < R ? wt[my] : 0.f;
    int j = 0;
    for (; j + U <= n; j += U) {
      u32x4 buf[U][NVL];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int row = __builtin_amdgcn_readlane(my_idx, j + u);
        const char* base = Vb + size_t(uint32_t(row)) * row_bytes;
#pragma unroll
        for (int m = 0; m < NVL; ++m) buf[u][m] = valid[m] ? ld16_nt(base + voff[m]) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j + u));
#pragma unroll
        for (int m = 0; m < NVL; ++m) {
          float f[E];
          Vec16<T>::widen(buf[u][m], f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[m][e] = fmaf(wf, f[e], acc[m][e]);
        }
      }
    }
    for (; j < n; ++j) {
      const int row = __builtin_amdgcn_readlane(my_idx, j);
      const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j));
      const char* base = Vb + size_t(uint32_t(row)) * row_bytes;
#pragma unroll
      for (int m = 0; m < NVL; ++m) {
        if (valid[m]) {
          float f[E];
          Vec16<T>::widen(ld16_nt(base + voff[m]), f);
#pragma unroll
          for (int e = 0; e < E; ++e) acc[m][e] = fmaf(wf, f[e], acc[m][e]);
        }
      }
    }
  }
  char* yb = reinterpret_cast<char*>(y) + size_t(t) * row_bytes;
#pragma unroll
  for (int m = 0; m < NVL; ++m)
    if (valid[m]) st16(yb + voff[m], Vec16<T>::narrow(acc[m]));
}

template <typename T, int NVL>
static void launch_gather_nvl(hipStream_t s, const int32_t* idx, const float* w, const void* V, void* y,
                              int64_t ntok, int R, int nvec) {
  constexpr int U = NVL <= 2 ? 8 : 4;
  dim3 grid(unsigned((ntok + 3) / 4), unsigned((nvec + 64 * NVL - 1) / (64 * NVL)));
  hipLaunchKernelGGL((gather_sum_kernel<T, NVL, U>), grid, dim3(256), 0, s, idx, w,
                     static_cast<const T*>(V), static_cast<T*>(y), ntok, R, nvec);
}

template <typename T>
static void launch_gather_t(hipStream_t s, const int32_t* idx, const float* w, const void* V, void* y,
                            int64_t ntok, int R, int nvec) {
  // Vectors per lane: enough to cover a row in one column block when the row
  // is at most 256 vectors (4 KB); wider rows use several column blocks.
  const int per_lane = (nvec + 63) / 64;
  if (per_lane <= 1)
    launch_gather_nvl<T, 1>(s, idx, w, V, y, ntok, R, nvec);
  else if (per_lane == 2)
    launch_gather_nvl<T, 2>(s, idx, w, V, y, ntok, R, nvec);
  else if (per_lane == 3)
    launch_gather_nvl<T, 3>(s, idx, w, V, y, ntok, R, nvec);
  else
    launch_gather_nvl<T, 4>(s, idx, w, V, y, ntok, R, nvec);
}

hipError_t launch_gather(hipStream_t s, int dtype, const int32_t* idx, const float* w, const void* V,
                         void* y, int64_t ntok, int R, int d_value) {
  const int elem = dtype == kBF16 ? 2 : 4;
  const int nvec = d_value * elem / 16;
  if (dtype == kBF16)
    launch_gather_t<bf16_t>(s, idx, w, V, y, ntok, R, nvec);
  else
    launch_gather_t<float>(s, idx, w, V, y, ntok, R, nvec);
  return hipGetLastError();
}

}  // namespace pkm
