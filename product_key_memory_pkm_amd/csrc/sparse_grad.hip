// Sparse backward (steps a7, a8, a9): gradient flows only through the
// selected rows and sub-keys ("Meta AI 可扩展内存层", section 6.1: only the
// activated key/value pairs accumulate gradient; section 9.2: back-propagate
// only at the selected positions; product-key paper summary, method details:
// only a few memory slots are updated).
//
//   dw[t,h,s] = <dY[t], V[r]>                       r = idx[t,h,s]
//   dV[r]    (+)= sum_{(t,h,s): idx = r} w[t,h,s] dY[t]
//   ds       = w (dw - sum_s w dw) / tau
//   dq1[t,h] = sum_s ds C[h, r/|C'|],  dq2[t,h] = sum_s ds C'[h, r%|C'|]
//   dC[h,i]  = sum_{(t,s): r/|C'| = i} ds q1[t,h],  likewise dC'
//
// value_grad walks the lookups grouped by row (a stable sort of the row ids),
// one wave per touched row: V[r] is read once and kept in registers, every
// lookup of r reads its dY row, produces dw with one wave reduction and adds
// w*dY into the row's fp32 gradient, which is written (or added) once.  The
// sub-key gradients use the same grouping keyed by sub-key.  Sums run in
// lookup order, so results are bit-identical from run to run.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int kVgU = 4;

template <typename T, int NVL>
__global__ __launch_bounds__(256) void value_grad_kernel(const int32_t* __restrict__ seg_start,
                                                         const int64_t* __restrict__ nseg_p,
                                                         const uint32_t* __restrict__ sorted_rows,
                                                         const int32_t* __restrict__ sorted_c,
                                                         const float* __restrict__ w, const T* __restrict__ dY,
                                                         const T* __restrict__ V, float* __restrict__ dV,
                                                         float* __restrict__ dw, int R, int nvec, int accumulate) {
  constexpr int E = Vec16<T>::N;
  const int lane = lane_id();
  const int64_t nseg = *nseg_p;
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const size_t row_bytes = size_t(nvec) * 16;
  const int dv = nvec * E;
  const char* Vb = reinterpret_cast<const char*>(V);
  const char* Yb = reinterpret_cast<const char*>(dY);

  bool valid[NVL];
  int voff[NVL];
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int v = m * 64 + lane;
    valid[m] = v < nvec;
    voff[m] = v * 16;
  }

  for (int64_t u = gw; u < nseg; u += nw) {
    const int lo = seg_start[u], hi = seg_start[u + 1];
    const uint32_t r = sorted_rows[lo];
    float vr[NVL][E], g[NVL][E];
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const u32x4 raw = valid[m] ? ld16_nt(Vb + size_t(r) * row_bytes + voff[m]) : u32x4{0, 0, 0, 0};
      Vec16<T>::widen(raw, vr[m]);
#pragma unroll
      for (int e = 0; e < E; ++e) g[m][e] = 0.f;
    }
    for (int c0 = lo; c0 < hi; c0 += 64) {
      const int n = min(64, hi - c0);
      const int my_c = lane < n ? sorted_c[c0 + lane] : 0;
      const float my_w = lane < n ? w[my_c] : 0.f;
      float my_dw = 0.f;
      int j = 0;
      for (; j < n; j += kVgU) {
        u32x4 buf[kVgU][NVL];
#pragma unroll
        for (int uu = 0; uu < kVgU; ++uu) {
          const int jj = j + uu < n ? j + uu : n - 1;
          const int c = __builtin_amdgcn_readlane(my_c, jj);
          const char* yrow = Yb + size_t(c / R) * row_bytes;
#pragma unroll
          for (int m = 0; m < NVL; ++m) buf[uu][m] = valid[m] ? ld16(yrow + voff[m]) : u32x4{0, 0, 0, 0};
        }
#pragma unroll
        for (int uu = 0; uu < kVgU; ++uu) {
          if (j + uu < n) {  // wave-uniform
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j + uu));
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < NVL; ++m) {
              float f[E];
              Vec16<T>::widen(buf[uu][m], f);
#pragma unroll
              for (int e = 0; e < E; ++e) {
                part = fmaf(f[e], vr[m][e], part);
                g[m][e] = fmaf(wt, f[e], g[m][e]);
              }
            }
            const float s = wave_sum(part);
            if (lane == j + uu) my_dw = s;
          }
        }
      }
      if (lane < n) dw[my_c] = my_dw;
    }
    float* drow = dV + size_t(r) * dv;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      if (!valid[m]) continue;
      float* p = drow + (m * 64 + lane) * E;
#pragma unroll
      for (int q4 = 0; q4 < E / 4; ++q4) {
        f32x4 o = {g[m][q4 * 4 + 0], g[m][q4 * 4 + 1], g[m][q4 * 4 + 2], g[m][q4 * 4 + 3]};
        if (accumulate) {
          const f32x4 old = *reinterpret_cast<const f32x4*>(p + q4 * 4);
          o += old;
        }
        *reinterpret_cast<f32x4*>(p + q4 * 4) = o;
      }
    }
  }
}

// 4 consecutive storage elements widened to fp32.
__device__ __forceinline__ void load4(const bf16_t* p, float* f) {
  const u32x2 v = *reinterpret_cast<const u32x2*>(p);
  f[0] = bf16lo(v.x); f[1] = bf16hi(v.x); f[2] = bf16lo(v.y); f[3] = bf16hi(v.y);
}
__device__ __forceinline__ void load4(const float* p, float* f) {
  const f32x4 v = *reinterpret_cast<const f32x4*>(p);
  f[0] = v.x; f[1] = v.y; f[2] = v.z; f[3] = v.w;
}

template <typename T>
__global__ __launch_bounds__(256) void softmax_bwd_dq_kernel(const int32_t* __restrict__ idx,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ dw, const T* __restrict__ C,
                                                             const T* __restrict__ Cp, int64_t nitems, int heads,
                                                             int dq, int k, int nk, int nk2, float inv_tau,
                                                             float* __restrict__ ds, float* __restrict__ dq_out) {
  const int lane = lane_id();
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int half = dq / 2;
  const int nch = half / 4;
  const int F = heads * dq;
  for (int64_t it = gw; it < nitems; it += nw) {
    const int hh = int(it % heads);
    const int64_t t = it / heads;
    const float wv = lane < k ? w[it * k + lane] : 0.f;
    const float dwv = lane < k ? dw[it * k + lane] : 0.f;
    const int row = lane < k ? idx[it * k + lane] : 0;
    const float sum = wave_sum(wv * dwv);
    const float dsv = lane < k ? wv * (dwv - sum) * inv_tau : 0.f;
    if (lane < k) ds[it * k + lane] = dsv;
    const int i = row / nk2;
    const int j = row - i * nk2;
    const T* Ch = C + size_t(hh) * nk * half;
    const T* Cph = Cp + size_t(hh) * nk2 * half;
    for (int ch = lane; ch - lane < nch; ch += 64) {
      const bool ok = ch < nch;
      float a1[4] = {0.f, 0.f, 0.f, 0.f}, a2[4] = {0.f, 0.f, 0.f, 0.f};
      for (int s = 0; s < k; ++s) {
        const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dsv), s));
        const int is = __builtin_amdgcn_readlane(i, s);
        const int js = __builtin_amdgcn_readlane(j, s);
        if (ok) {
          float c1[4], c2[4];
          load4(Ch + size_t(is) * half + ch * 4, c1);
          load4(Cph + size_t(js) * half + ch * 4, c2);
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            a1[e] = fmaf(d, c1[e], a1[e]);
            a2[e] = fmaf(d, c2[e], a2[e]);
          }
        }
      }
      if (ok) {
        float* o = dq_out + size_t(t) * F + size_t(hh) * dq + ch * 4;
        *reinterpret_cast<f32x4*>(o) = f32x4{a1[0], a1[1], a1[2], a1[3]};
        *reinterpret_cast<f32x4*>(o + half) = f32x4{a2[0], a2[1], a2[2], a2[3]};
      }
    }
  }
}

__global__ __launch_bounds__(256) void subkey_keys_kernel(const int32_t* __restrict__ idx, int64_t n, int heads,
                                                          int k, int nk, int nk2, int half_sel,
                                                          uint32_t* __restrict__ keys) {
  for (int64_t c = int64_t(blockIdx.x) * 256 + threadIdx.x; c < n; c += int64_t(gridDim.x) * 256) {
    const uint32_t hh = uint32_t((c / k) % heads);
    const int row = idx[c];
    keys[c] = half_sel ? hh * uint32_t(nk2) + uint32_t(row % nk2) : hh * uint32_t(nk) + uint32_t(row / nk2);
  }
}

constexpr int kSkU = 8;

template <typename T>
__global__ __launch_bounds__(256) void subkey_grad_kernel(const int32_t* __restrict__ seg_start,
                                                          const int64_t* __restrict__ nseg_p,
                                                          const uint32_t* __restrict__ sorted_keys,
                                                          const int32_t* __restrict__ sorted_c,
                                                          const float* __restrict__ ds, const T* __restrict__ q,
                                                          int heads, int dq, int k, int half_sel, int nkeys,
                                                          float* __restrict__ dC) {
  const int lane = lane_id();
  const int64_t nseg = *nseg_p;
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int half = dq / 2;
  const int nch = half / 4;
  const int F = heads * dq;
  for (int64_t u = gw; u < nseg; u += nw) {
    const int lo = seg_start[u], hi = seg_start[u + 1];
    const uint32_t key = sorted_keys[lo];
    const int hh = int(key / uint32_t(nkeys));
    const T* qh = q + size_t(hh) * dq + size_t(half_sel) * half;
    for (int chb = 0; chb < nch; chb += 64) {
      const int ch = chb + lane;
      const bool ok = ch < nch;
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = lo; c0 < hi; c0 += 64) {
        const int n = min(64, hi - c0);
        const int my_c = lane < n ? sorted_c[c0 + lane] : 0;
        const float my_ds = lane < n ? ds[my_c] : 0.f;
        for (int j = 0; j < n; j += kSkU) {
          float f[kSkU][4];
#pragma unroll
          for (int uu = 0; uu < kSkU; ++uu) {
            const int jj = j + uu < n ? j + uu : n - 1;
            const int c = __builtin_amdgcn_readlane(my_c, jj);
            const int64_t t = int64_t(c / k) / heads;
            if (ok) load4(qh + size_t(t) * F + ch * 4, f[uu]);
          }
#pragma unroll
          for (int uu = 0; uu < kSkU; ++uu) {
            if (j + uu < n && ok) {
              const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_ds), j + uu));
#pragma unroll
              for (int e = 0; e < 4; ++e) a[e] = fmaf(d, f[uu][e], a[e]);
            }
          }
        }
      }
      if (ok) *reinterpret_cast<f32x4*>(dC + size_t(key) * half + ch * 4) = f32x4{a[0], a[1], a[2], a[3]};
    }
  }
}

inline unsigned grid_waves(int64_t items, int64_t cap_blocks = 4096) {
  int64_t b = (items + 3) / 4;
  if (b > cap_blocks) b = cap_blocks;
  if (b < 1) b = 1;
  return unsigned(b);
}

}  // namespace

hipError_t launch_value_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg,
                             int64_t nitems, const uint32_t* sorted_rows, const int32_t* sorted_c, const float* w,
                             const void* dY, const void* V, float* dV, float* dw, int R, int d_value,
                             bool accumulate) {
  const int elem = dtype == kBF16 ? 2 : 4;
  const int nvec = d_value * elem / 16;
  const int per_lane = (nvec + 63) / 64;
  const dim3 grid(grid_waves(nitems)), block(256);
#define PKM_VG(TT, NV)                                                                                        \
  hipLaunchKernelGGL((value_grad_kernel<TT, NV>), grid, block, 0, s, seg_start, nseg, sorted_rows, sorted_c, w, \
                     static_cast<const TT*>(dY), static_cast<const TT*>(V), dV, dw, R, nvec, int(accumulate))
  if (dtype == kBF16) {
    if (per_lane <= 1) PKM_VG(bf16_t, 1);
    else if (per_lane == 2) PKM_VG(bf16_t, 2);
    else if (per_lane == 3) PKM_VG(bf16_t, 3);
    else if (per_lane == 4) PKM_VG(bf16_t, 4);
    else return hipErrorInvalidValue;
  } else {
    if (per_lane <= 1) PKM_VG(float, 1);
    else if (per_lane == 2) PKM_VG(float, 2);
    else if (per_lane == 3) PKM_VG(float, 3);
    else if (per_lane == 4) PKM_VG(float, 4);
    else return hipErrorInvalidValue;
  }
#undef PKM_VG
  return hipGetLastError();
}

hipError_t launch_softmax_bwd_dq(hipStream_t s, int dtype, const int32_t* idx, const float* w, const float* dw,
                                 const void* C, const void* Cp, int64_t ntok, int heads, int dq, int k, int nk,
                                 int nk2, float inv_tau, float* ds, float* dq_out) {
  const int64_t nitems = ntok * heads;
  const dim3 grid(grid_waves(nitems, 8192)), block(256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(softmax_bwd_dq_kernel<bf16_t>, grid, block, 0, s, idx, w, dw, static_cast<const bf16_t*>(C),
                       static_cast<const bf16_t*>(Cp), nitems, heads, dq, k, nk, nk2, inv_tau, ds, dq_out);
  else
    hipLaunchKernelGGL(softmax_bwd_dq_kernel<float>, grid, block, 0, s, idx, w, dw, static_cast<const float*>(C),
                       static_cast<const float*>(Cp), nitems, heads, dq, k, nk, nk2, inv_tau, ds, dq_out);
  return hipGetLastError();
}

hipError_t launch_subkey_keys(hipStream_t s, const int32_t* idx, int64_t n, int heads, int k, int nk, int nk2,
                              int half_sel, uint32_t* keys) {
  int64_t b = (n + 255) / 256;
  if (b > 16384) b = 16384;
  if (b < 1) b = 1;
  hipLaunchKernelGGL(subkey_keys_kernel, dim3(unsigned(b)), dim3(256), 0, s, idx, n, heads, k, nk, nk2, half_sel,
                     keys);
  return hipGetLastError();
}

hipError_t launch_subkey_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg, int64_t nitems,
                              const uint32_t* sorted_keys, const int32_t* sorted_c, const float* ds, const void* q,
                              int heads, int dq, int k, int half_sel, int nkeys, float* dC) {
  const dim3 grid(grid_waves(nitems)), block(256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(subkey_grad_kernel<bf16_t>, grid, block, 0, s, seg_start, nseg, sorted_keys, sorted_c, ds,
                       static_cast<const bf16_t*>(q), heads, dq, k, half_sel, nkeys, dC);
  else
    hipLaunchKernelGGL(subkey_grad_kernel<float>, grid, block, 0, s, seg_start, nseg, sorted_keys, sorted_c, ds,
                       static_cast<const float*>(q), heads, dq, k, half_sel, nkeys, dC);
  return hipGetLastError();
}

}  // namespace pkm
