// Steps a5 + a6 in one launch for the forward: the k x k candidate merge and
// softmax of every head of a token, then the softmax-weighted sum of the
// selected value rows ("Meta AI 可扩展内存层", sections 4.3, 4.5, 5.3 and 9.2;
// product-key paper summary, method details).
#include "common.h"
#include "kernels.h"
#include "merge_common.h"

namespace pkm {

namespace {

// Steps a5 + a6 fused for the forward: one wave per token merges its heads'
// candidate lists (merge_item, the arithmetic of the merge kernel), writes the
// rows and weights the backward keeps, and gathers the value rows of each
// 64-row chunk (64 / k heads) with the loop of gather_sum_kernel, rows in the
// same order, so y is bit-identical to the two launches.  The merge's VALU
// work runs while the other waves' row loads are in flight.  resid != null
// (the fast-weight memorization): also the residual y - target, as
// gather_sum_kernel writes it.
template <typename T, int NVL, int U>
__global__ __launch_bounds__(256) void merge_gather_kernel(const int32_t* __restrict__ sub_idx,
                                                           const float* __restrict__ sub_score, int64_t ntok,
                                                           int heads, int k, int nk2, float inv_tau,
                                                           int32_t* __restrict__ idx_out, float* __restrict__ w_out,
                                                           const T* __restrict__ V, T* __restrict__ y, int nvec,
                                                           const T* __restrict__ target, T* __restrict__ resid) {
  constexpr int E = Vec16<T>::N;
  __shared__ uint16_t pairs[128];
  __shared__ int npairs;
  __shared__ uint64_t scratch[4][64];
  merge_build_pairs(k, pairs, &npairs);
  __syncthreads();
  const int lane = lane_id();
  const int wave = threadIdx.x >> 6;
  const int64_t t = int64_t(blockIdx.x) * 4 + wave;
  if (t >= ntok) return;
  const MergeLanePairs lp = merge_lane_pairs(pairs, npairs);
  const size_t row_bytes = size_t(nvec) * 16;
  const char* Vb = reinterpret_cast<const char*>(V);
  bool valid[NVL];
  int voff[NVL];
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int v = m * 64 + lane;
    valid[m] = v < nvec;
    voff[m] = v * 16;
  }
  float acc[NVL][E];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int e = 0; e < E; ++e) acc[m][e] = 0.f;

  const int hpc = 64 / k;  // heads per 64-row chunk
  for (int h0 = 0; h0 < heads; h0 += hpc) {
    const int nh = heads - h0 < hpc ? heads - h0 : hpc;
    int my_idx = 0;
    float my_w = 0.f;
    for (int qh = 0; qh < nh; ++qh) {
      const int64_t it = t * heads + h0 + qh;
      int row;
      float wv, sc;
      merge_item(sub_idx, sub_score, it, k, nk2, inv_tau, lp, scratch[wave], row, wv, sc);
      if (lane < k) {
        idx_out[it * k + lane] = row;
        w_out[it * k + lane] = wv;
      }
      // slot s of this head goes to lane qh k + s of the chunk
      const int src = (lane - qh * k) & 63;
      const int r2 = __shfl(row, src, 64);
      const float w2 = __shfl(wv, src, 64);
      if (lane >= qh * k && lane < (qh + 1) * k) {
        my_idx = r2;
        my_w = w2;
      }
    }
    const int n = nh * k;
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
  if (resid) {  // wave-uniform
    const char* tb = reinterpret_cast<const char*>(target) + size_t(t) * row_bytes;
    char* eb = reinterpret_cast<char*>(resid) + size_t(t) * row_bytes;
#pragma unroll
    for (int m = 0; m < NVL; ++m)
      if (valid[m]) {
        float yf[E], tf[E];
        Vec16<T>::widen(Vec16<T>::narrow(acc[m]), yf);
        Vec16<T>::widen(ld16(tb + voff[m]), tf);
#pragma unroll
        for (int e = 0; e < E; ++e) yf[e] -= tf[e];
        st16(eb + voff[m], Vec16<T>::narrow(yf));
      }
  }
}

}  // namespace

template <typename T, int NVL>
static void launch_merge_gather_nvl(hipStream_t s, const int32_t* sub_idx, const float* sub_score, int64_t ntok,
                                    int heads, int k, int nk2, float inv_tau, int32_t* idx, float* w, const void* V,
                                    void* y, int nvec, const void* target, void* resid) {
  constexpr int U = NVL <= 2 ? 8 : 4;
  hipLaunchKernelGGL((merge_gather_kernel<T, NVL, U>), dim3(unsigned((ntok + 3) / 4)), dim3(256), 0, s, sub_idx,
                     sub_score, ntok, heads, k, nk2, inv_tau, idx, w, static_cast<const T*>(V), static_cast<T*>(y),
                     nvec, static_cast<const T*>(target), static_cast<T*>(resid));
}

template <typename T>
static void launch_merge_gather_t(hipStream_t s, const int32_t* sub_idx, const float* sub_score, int64_t ntok,
                                  int heads, int k, int nk2, float inv_tau, int32_t* idx, float* w, const void* V,
                                  void* y, int nvec, const void* target, void* resid) {
  const int per_lane = (nvec + 63) / 64;
  if (per_lane <= 1)
    launch_merge_gather_nvl<T, 1>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                  resid);
  else if (per_lane == 2)
    launch_merge_gather_nvl<T, 2>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                  resid);
  else if (per_lane == 3)
    launch_merge_gather_nvl<T, 3>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                  resid);
  else
    launch_merge_gather_nvl<T, 4>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                  resid);
}

bool merge_gather_supported(int dtype, int k, int d_value, bool fp8_values) {
  const int elem = dtype == kBF16 ? 2 : 4;
  return !fp8_values && k >= 1 && k <= 32 && 64 % k == 0 && (d_value * elem) % 16 == 0 &&
         d_value * elem / 16 <= 256;
}

hipError_t launch_merge_gather(hipStream_t s, int dtype, const int32_t* sub_idx, const float* sub_score, int64_t ntok,
                               int heads, int k, int nk2, float inv_tau, int32_t* idx, float* w, const void* V,
                               void* y, int d_value, bool fp8_values, const void* target, void* resid) {
  if (!merge_gather_supported(dtype, k, d_value, fp8_values)) return hipErrorInvalidValue;
  if ((resid == nullptr) != (target == nullptr)) return hipErrorInvalidValue;
  if (ntok == 0) return hipGetLastError();
  const int elem = dtype == kBF16 ? 2 : 4;
  const int nvec = d_value * elem / 16;
  if (dtype == kBF16)
    launch_merge_gather_t<bf16_t>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                  resid);
  else
    launch_merge_gather_t<float>(s, sub_idx, sub_score, ntok, heads, k, nk2, inv_tau, idx, w, V, y, nvec, target,
                                 resid);
  return hipGetLastError();
}

}  // namespace pkm
