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

constexpr int kVgU = 2;


// <a, v> over one 16-byte vector, accumulated into c.  bf16: v_dot2_f32_bf16 on
// packed pairs (products exact in fp32); fp32: four FMAs.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& v, float c);
template <>
__device__ __forceinline__ float dot16<bf16_t>(const u32x4& a, const u32x4& v, float c) {
  // whole-vector bit casts and shuffles: casting single elements of a u32x4 to
  // bf16x2 miscompiles here (every pair read the same register)
  const bf16x8 A = __builtin_bit_cast(bf16x8, a), B = __builtin_bit_cast(bf16x8, v);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 0, 1), __builtin_shufflevector(B, B, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 2, 3), __builtin_shufflevector(B, B, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 4, 5), __builtin_shufflevector(B, B, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 6, 7), __builtin_shufflevector(B, B, 6, 7), c, false);
  return c;
}
template <>
__device__ __forceinline__ float dot16<float>(const u32x4& a, const u32x4& v, float c) {
  c = fmaf(__uint_as_float(a.x), __uint_as_float(v.x), c);
  c = fmaf(__uint_as_float(a.y), __uint_as_float(v.y), c);
  c = fmaf(__uint_as_float(a.z), __uint_as_float(v.z), c);
  c = fmaf(__uint_as_float(a.w), __uint_as_float(v.w), c);
  return c;
}

// One wave per touched row (grid-stride over rows).  Lane l owns 16-byte
// vectors l, l+64, ... of the row; the first NVL-1 are in range for every lane
// (the launcher picks NVL so), only the last one is predicated: out-of-range
// lanes read vector 0 instead (discarded), so every load is issued unconditionally.  The value row stays in
// its storage format; each lookup costs one dY row read, NVL dot products, one
// DPP wave reduction and the fp32 FMAs of w*dY.
template <typename T, int NVL>
__global__ __launch_bounds__(256) void value_grad_kernel(const int32_t* __restrict__ seg_start,
                                                         const int64_t* __restrict__ nseg_p,
                                                         const uint32_t* __restrict__ sorted_rows,
                                                         const int32_t* __restrict__ sorted_c,
                                                         const float* __restrict__ w, const T* __restrict__ dY,
                                                         const T* __restrict__ V, float* __restrict__ dV,
                                                         float* __restrict__ dw, uint32_t R, int nvec, int accumulate) {
  constexpr int E = Vec16<T>::N;
  const int lane = lane_id();
  const int64_t nseg = *nseg_p;
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const size_t row_bytes = size_t(nvec) * 16;
  const int dv = nvec * E;
  const char* Vb = reinterpret_cast<const char*>(V);
  const char* Yb = reinterpret_cast<const char*>(dY);
  const bool last_ok = (NVL - 1) * 64 + lane < nvec;
  int voff[NVL];
#pragma unroll
  for (int m = 0; m < NVL; ++m) voff[m] = (m < NVL - 1 || last_ok) ? (m * 64 + lane) * 16 : 0;  // clamp to vector 0

  for (int64_t u = gw; u < nseg; u += nw) {
    const int lo = seg_start[u], hi = seg_start[u + 1];
    const uint32_t r = sorted_rows[lo];
    const char* vrow = Vb + size_t(r) * row_bytes;
    u32x4 vr[NVL];
    float g[NVL][E];
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      vr[m] = ld16_nt(vrow + voff[m]);
#pragma unroll
      for (int e = 0; e < E; ++e) g[m][e] = 0.f;
    }
    if (!last_ok) vr[NVL - 1] = u32x4{0, 0, 0, 0};
    for (int c0 = lo; c0 < hi; c0 += 64) {
      const int n = min(64, hi - c0);
      const int my_c = lane < n ? sorted_c[c0 + lane] : 0;
      const float my_w = lane < n ? w[my_c] : 0.f;
      float my_dw = 0.f;
      for (int j = 0; j < n; j += kVgU) {
        u32x4 buf[kVgU][NVL];
#pragma unroll
        for (int uu = 0; uu < kVgU; ++uu) {
          const int jj = j + uu < n ? j + uu : n - 1;
          const uint32_t c = uint32_t(__builtin_amdgcn_readlane(my_c, jj));
          const char* yrow = Yb + size_t(c / R) * row_bytes;
#pragma unroll
          for (int m = 0; m < NVL; ++m) buf[uu][m] = ld16(yrow + voff[m]);
        }
#pragma unroll
        for (int uu = 0; uu < kVgU; ++uu) {
          if (j + uu < n) {  // wave-uniform
            const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j + uu));
            float part = 0.f;
#pragma unroll
            for (int m = 0; m < NVL; ++m) {
              part = dot16<T>(buf[uu][m], vr[m], part);
              float f[E];
              Vec16<T>::widen(buf[uu][m], f);
#pragma unroll
              for (int e = 0; e < E; ++e) g[m][e] = fmaf(wt, f[e], g[m][e]);
            }
            const float s = wave_sum_dpp(part);
            if (lane == j + uu) my_dw = s;
          }
        }
      }
      if (lane < n) dw[my_c] = my_dw;
    }
    float* drow = dV + size_t(r) * dv;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      if (m == NVL - 1 && !last_ok) continue;
      float* p = drow + (voff[m] / 16) * E;
#pragma unroll
      for (int q4 = 0; q4 < E / 4; ++q4) {
        f32x4 o = {g[m][q4 * 4 + 0], g[m][q4 * 4 + 1], g[m][q4 * 4 + 2], g[m][q4 * 4 + 3]};
        if (accumulate) o += *reinterpret_cast<const f32x4*>(p + q4 * 4);
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
__device__ __forceinline__ void load4_acc(const T* p, float d, float* a) {
  float f[4];
  load4(p, f);
#pragma unroll
  for (int e = 0; e < 4; ++e) a[e] = fmaf(d, f[e], a[e]);
}

// One wave per (token, head):
//  * softmax backward ds = w (dw - sum w dw) / tau over the k selected slots;
//  * the k slots name k (i, j) sub-key pairs with repeats; the coefficient of
//    each distinct i (j) is the sum of ds over its slots, and only distinct
//    sub-keys are read: dq1 = sum_i coef_i C[h,i], dq2 = sum_j coef_j C'[h,j];
//  * for the sub-key gradients, slot s gets key h*|C|+i (or h*|C'|+j) and the
//    coefficient when it is the first slot of its sub-key, else a sentinel key
//    that sorts after every real one.
template <typename T>
__global__ __launch_bounds__(256) void softmax_bwd_dq_kernel(const int32_t* __restrict__ idx,
                                                             const float* __restrict__ w,
                                                             const float* __restrict__ dw, const T* __restrict__ C,
                                                             const T* __restrict__ Cp, int64_t nitems, int heads,
                                                             int dq, int k, int nk, int nk2, float inv_tau,
                                                             float* __restrict__ dq_out, uint32_t* __restrict__ key1,
                                                             float* __restrict__ coef1, uint32_t* __restrict__ key2,
                                                             float* __restrict__ coef2) {
  const int lane = lane_id();
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int half = dq / 2;
  const int nch = half / 4;
  const int F = heads * dq;
  const uint32_t sent1 = uint32_t(heads) * uint32_t(nk), sent2 = uint32_t(heads) * uint32_t(nk2);
  for (int64_t it = gw; it < nitems; it += nw) {
    const int hh = int(it % heads);
    const int64_t t = it / heads;
    const bool act = lane < k;
    const float wv = act ? w[it * k + lane] : 0.f;
    const float dwv = act ? dw[it * k + lane] : 0.f;
    const int row = act ? idx[it * k + lane] : 0;
    const float sum = wave_sum_dpp(wv * dwv);
    const float dsv = act ? wv * (dwv - sum) * inv_tau : 0.f;
    const int i = row / nk2;
    const int j = row - i * nk2;
    float s1 = 0.f, s2 = 0.f;
    bool dup1 = false, dup2 = false;
    for (int sp = 0; sp < k; ++sp) {
      const int is = __builtin_amdgcn_readlane(i, sp);
      const int js = __builtin_amdgcn_readlane(j, sp);
      const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(dsv), sp));
      if (i == is) {
        s1 += d;
        dup1 |= sp < lane;
      }
      if (j == js) {
        s2 += d;
        dup2 |= sp < lane;
      }
    }
    const bool first1 = act && !dup1, first2 = act && !dup2;
    if (act) {
      const int64_t c = it * k + lane;
      key1[c] = first1 ? uint32_t(hh) * uint32_t(nk) + uint32_t(i) : sent1;
      coef1[c] = s1;
      key2[c] = first2 ? uint32_t(hh) * uint32_t(nk2) + uint32_t(j) : sent2;
      coef2[c] = s2;
    }
    const uint64_t m1 = ballot(first1), m2 = ballot(first2);
    const T* Ch = C + size_t(hh) * nk * half;
    const T* Cph = Cp + size_t(hh) * nk2 * half;
    float* o = dq_out + size_t(t) * F + size_t(hh) * dq;
    for (int chb = 0; chb < nch; chb += 64) {
      const int ch = min(chb + lane, nch - 1);  // clamped; the store below is predicated
      float a1[4] = {0.f, 0.f, 0.f, 0.f}, a2[4] = {0.f, 0.f, 0.f, 0.f};
      uint64_t mm = m1;
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        const int is = __builtin_amdgcn_readlane(i, b);
        load4_acc(Ch + size_t(is) * half + ch * 4, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), b)), a1);
      }
      mm = m2;
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        const int js = __builtin_amdgcn_readlane(j, b);
        load4_acc(Cph + size_t(js) * half + ch * 4, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s2), b)), a2);
      }
      if (chb + lane < nch) {
        *reinterpret_cast<f32x4*>(o + ch * 4) = f32x4{a1[0], a1[1], a1[2], a1[3]};
        *reinterpret_cast<f32x4*>(o + half + ch * 4) = f32x4{a2[0], a2[1], a2[2], a2[3]};
      }
    }
  }
}

constexpr int kSkU = 8;
constexpr int kSkWaves = 4;

// One 4-wave block per sub-key (grid-stride): dC[key] = sum over its entries of
// coef * q_half[t, h].  Wave v takes entries v, v+4, ... in batches of 8 rows,
// and the four partial sums are added in wave order through LDS.
template <typename T>
__global__ __launch_bounds__(256) void subkey_grad_kernel(const int32_t* __restrict__ seg_start,
                                                          const int64_t* __restrict__ nseg_p,
                                                          const uint32_t* __restrict__ sorted_keys,
                                                          const int32_t* __restrict__ sorted_c,
                                                          const float* __restrict__ coef, const T* __restrict__ q,
                                                          int heads, int dq, int k, int half_sel, int nkeys,
                                                          float* __restrict__ dC) {
  __shared__ f32x4 part[kSkWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int64_t nseg = *nseg_p;
  const int half = dq / 2;
  const int nch = half / 4;
  const int F = heads * dq;
  const uint32_t nvalid = uint32_t(heads) * uint32_t(nkeys);
  const int kh = k * heads;
  for (int64_t u = blockIdx.x; u < nseg; u += gridDim.x) {
    const int lo = seg_start[u], hi = seg_start[u + 1];
    const uint32_t key = sorted_keys[lo];
    if (key >= nvalid) continue;  // block-uniform: the sentinel run (repeated sub-keys)
    const int hh = int(key / uint32_t(nkeys));
    const T* qh = q + size_t(hh) * dq + size_t(half_sel) * half;
    for (int chb = 0; chb < nch; chb += 64) {
      const int ch = min(chb + lane, nch - 1);
      float a[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = lo + wave; c0 < hi; c0 += kSkWaves * 64) {
        // entries c0, c0+4, ..., one per lane
        const int e = c0 + lane * kSkWaves;
        const int my_c = e < hi ? sorted_c[e] : 0;
        const float my_d = e < hi ? coef[my_c] : 0.f;
        const int n = min(64, (hi - c0 + kSkWaves - 1) / kSkWaves);
        for (int jb = 0; jb < n; jb += kSkU) {
          float f[kSkU][4];
#pragma unroll
          for (int uu = 0; uu < kSkU; ++uu) {
            const int jj = jb + uu < n ? jb + uu : n - 1;
            const uint32_t c = uint32_t(__builtin_amdgcn_readlane(my_c, jj));
            load4(qh + size_t(c / uint32_t(kh)) * F + ch * 4, f[uu]);
          }
#pragma unroll
          for (int uu = 0; uu < kSkU; ++uu) {
            if (jb + uu < n) {
              const float d = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_d), jb + uu));
#pragma unroll
              for (int q4 = 0; q4 < 4; ++q4) a[q4] = fmaf(d, f[uu][q4], a[q4]);
            }
          }
        }
      }
      part[wave][lane] = f32x4{a[0], a[1], a[2], a[3]};
      __syncthreads();
      if (wave == 0 && chb + lane < nch) {
        f32x4 tot = part[0][lane];
#pragma unroll
        for (int v = 1; v < kSkWaves; ++v) tot += part[v][lane];
        *reinterpret_cast<f32x4*>(dC + size_t(key) * half + ch * 4) = tot;
      }
      __syncthreads();
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
                     static_cast<const TT*>(dY), static_cast<const TT*>(V), dV, dw, uint32_t(R), nvec,          \
                     int(accumulate))
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
                                 int nk2, float inv_tau, float* dq_out, uint32_t* key1, float* coef1, uint32_t* key2,
                                 float* coef2) {
  const int64_t nitems = ntok * heads;
  const dim3 grid(grid_waves(nitems, 8192)), block(256);
  if (dtype == kBF16)
    hipLaunchKernelGGL(softmax_bwd_dq_kernel<bf16_t>, grid, block, 0, s, idx, w, dw, static_cast<const bf16_t*>(C),
                       static_cast<const bf16_t*>(Cp), nitems, heads, dq, k, nk, nk2, inv_tau, dq_out, key1, coef1,
                       key2, coef2);
  else
    hipLaunchKernelGGL(softmax_bwd_dq_kernel<float>, grid, block, 0, s, idx, w, dw, static_cast<const float*>(C),
                       static_cast<const float*>(Cp), nitems, heads, dq, k, nk, nk2, inv_tau, dq_out, key1, coef1,
                       key2, coef2);
  return hipGetLastError();
}

hipError_t launch_subkey_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg, int64_t nsub,
                              const uint32_t* sorted_keys, const int32_t* sorted_c, const float* coef, const void* q,
                              int heads, int dq, int k, int half_sel, int nkeys, float* dC) {
  int64_t blocks = nsub + 1;  // at most one block per distinct sub-key (+ the sentinel run)
  if (blocks > 8192) blocks = 8192;
  const dim3 grid{unsigned(blocks), 1, 1}, block{256, 1, 1};
  if (dtype == kBF16)
    hipLaunchKernelGGL(subkey_grad_kernel<bf16_t>, grid, block, 0, s, seg_start, nseg, sorted_keys, sorted_c, coef,
                       static_cast<const bf16_t*>(q), heads, dq, k, half_sel, nkeys, dC);
  else
    hipLaunchKernelGGL(subkey_grad_kernel<float>, grid, block, 0, s, seg_start, nseg, sorted_keys, sorted_c, coef,
                       static_cast<const float*>(q), heads, dq, k, half_sel, nkeys, dC);
  return hipGetLastError();
}

}  // namespace pkm
