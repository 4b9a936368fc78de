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
//  * fp32 accumulation in registers, one rounding to the storage type;
//  * optionally (the fast-weight memorization) the residual y - target, from y
//    as stored and rounded once more, written beside y.
#include "common.h"
#include "kernels.h"

namespace pkm {

template <typename T, int NVL, int U>
__global__ __launch_bounds__(256) void gather_sum_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const T* __restrict__ V, T* __restrict__ y,
                                                         int64_t ntok, int R, int nvec,
                                                         const T* __restrict__ target, T* __restrict__ resid) {
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

// ---------------------------------------------------------------------------
// fp8 value rows ("Meta AI 可扩展内存层", section 16.3: the value table stored
// in a low-bit format).  Row r takes d_value + 16 bytes rounded up to a
// multiple of 128 (whole 128-byte lines): a 16-byte header whose first 4 bytes
// are the fp32 scale s_r, then d_value E4M3 codes (1 sign, 4 exponent bits with
// bias 7, 3 mantissa bits), then zeros; the value is s_r * code.
// ---------------------------------------------------------------------------
constexpr float kE4M3Max = 448.f;

// 16 codes of one 16-byte vector -> fp32 (hardware pair conversions; every
// E4M3 value is exact in fp32).
__device__ __forceinline__ void e4m3x16_to_f32(const u32x4& c, float* f) {
  const uint32_t wd[4] = {c.x, c.y, c.z, c.w};
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const auto lo = __builtin_amdgcn_cvt_pk_f32_fp8(int(wd[i]), false);  // bytes 0, 1
    const auto hi = __builtin_amdgcn_cvt_pk_f32_fp8(int(wd[i]), true);   // bytes 2, 3
    f[4 * i + 0] = lo[0];
    f[4 * i + 1] = lo[1];
    f[4 * i + 2] = hi[0];
    f[4 * i + 3] = hi[1];
  }
}

// Nearest E4M3 code of q (ties to the even code), |q| saturated at 448; zero
// (of either sign) gives code 0.  Subnormal steps are 2^-9; a normal value
// a = (1 + m/8) 2^e has code ((e + 7) << 3) + m, and a rounded-up mantissa of 8
// carries into the next exponent, which the code arithmetic does by itself.
__device__ __forceinline__ uint32_t f32_to_e4m3(float q) {
  const uint32_t sign = (__float_as_uint(q) >> 24) & 0x80u;
  float a = fminf(fabsf(q), kE4M3Max);
  uint32_t code;
  if (!(a > 0.f)) return 0u;
  if (a < 0.015625f) {  // below 2^-6: subnormal codes 0..8 (8 is the smallest normal)
    code = uint32_t(__builtin_rintf(a * 512.f));
  } else {
    const int e = int((__float_as_uint(a) >> 23) & 0xFF) - 127;  // -6 .. 8
    const float frac = __builtin_amdgcn_ldexpf(a, -e);            // [1, 2), exact
    code = uint32_t((e + 7) << 3) + uint32_t(__builtin_rintf((frac - 1.f) * 8.f));
  }
  code = code < 0x7Eu ? code : 0x7Eu;
  return code ? (code | sign) : 0u;
}

template <typename T, int NVL, int U>
__global__ __launch_bounds__(256) void gather_fp8_kernel(const int32_t* __restrict__ idx,
                                                         const float* __restrict__ w,
                                                         const uint8_t* __restrict__ V, T* __restrict__ y,
                                                         int64_t ntok, int R, int nvec) {
  constexpr int EO = Vec16<T>::N;  // output elements per 16-byte store
  const int lane = lane_id();
  const int64_t t = int64_t(blockIdx.x) * 4 + (threadIdx.x >> 6);
  if (t >= ntok) return;
  const size_t row_bytes = fp8_row_bytes(nvec);
  const char* Vb = reinterpret_cast<const char*>(V);
  bool valid[NVL];
  int voff[NVL];
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const int v = m * 64 + lane;  // this lane's 16-code vector
    valid[m] = v < nvec;
    voff[m] = 16 + v * 16;
  }
  float acc[NVL][16];
#pragma unroll
  for (int m = 0; m < NVL; ++m)
#pragma unroll
    for (int e = 0; e < 16; ++e) acc[m][e] = 0.f;
  const int32_t* it = idx + t * R;
  const float* wt = w + t * R;
  for (int r0 = 0; r0 < R; r0 += 64) {
    const int n = min(64, R - r0);
    const int my = r0 + lane;
    const int my_idx = my < R ? it[my] : 0;
    const float my_w = my < R ? wt[my] : 0.f;
    for (int j = 0; j < n; j += U) {
      u32x4 buf[U][NVL];
      float sc[U];
#pragma unroll
      for (int u = 0; u < U; ++u) {
        const int jj = j + u < n ? j + u : n - 1;
        const int row = __builtin_amdgcn_readlane(my_idx, jj);
        const char* base = Vb + size_t(uint32_t(row)) * row_bytes;
        sc[u] = *reinterpret_cast<const float*>(base);
#pragma unroll
        for (int m = 0; m < NVL; ++m) buf[u][m] = valid[m] ? ld16_nt(base + voff[m]) : u32x4{0, 0, 0, 0};
      }
#pragma unroll
      for (int u = 0; u < U; ++u) {
        if (j + u < n) {  // wave-uniform
          const float wf = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j + u)) * sc[u];
#pragma unroll
          for (int m = 0; m < NVL; ++m) {
            float f[16];
            e4m3x16_to_f32(buf[u][m], f);
#pragma unroll
            for (int e = 0; e < 16; ++e) acc[m][e] = fmaf(wf, f[e], acc[m][e]);
          }
        }
      }
    }
  }
  char* yb = reinterpret_cast<char*>(y) + size_t(t) * size_t(nvec) * 16 * sizeof(T);
#pragma unroll
  for (int m = 0; m < NVL; ++m)
    if (valid[m]) {
      char* dst = yb + size_t(m * 64 + lane) * 16 * sizeof(T);
#pragma unroll
      for (int q = 0; q < 16 / EO; ++q) st16(dst + q * 16, Vec16<T>::narrow(&acc[m][q * EO]));
    }
}

// One wave per row: the row's largest magnitude gives s = max / 448 and the
// factor 448 / max (both fp32); every element is stored as the nearest E4M3
// code of element * factor.  A zero row gets s = 0 and zero codes.
template <typename T, int NVL>
__global__ __launch_bounds__(256) void quantize_fp8_kernel(const T* __restrict__ src, int64_t rows, int nvec,
                                                           uint8_t* __restrict__ dst) {
  constexpr int EI = Vec16<T>::N;  // input elements per 16-byte load
  const int lane = lane_id();
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const size_t in_row = size_t(nvec) * 16 * sizeof(T);  // bytes of a source row
  const size_t out_row = fp8_row_bytes(nvec);
  const int npad = int((out_row - 16) / 16) - nvec;  // zero vectors after the codes
  for (int64_t r = gw; r < rows; r += nw) {
    const char* rs = reinterpret_cast<const char*>(src) + size_t(r) * in_row;
    float f[NVL][16];
    float mx = 0.f;
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int v = m * 64 + lane;
      if (v < nvec) {
#pragma unroll
        for (int q = 0; q < 16 / EI; ++q) Vec16<T>::widen(ld16(rs + size_t(v) * 16 * sizeof(T) + q * 16), &f[m][q * EI]);
      } else {
#pragma unroll
        for (int e = 0; e < 16; ++e) f[m][e] = 0.f;
      }
#pragma unroll
      for (int e = 0; e < 16; ++e) mx = fmaxf(mx, fabsf(f[m][e]));
    }
    mx = wave_max(mx);
    const float scale = mx > 0.f ? mx / kE4M3Max : 0.f;
    const float inv = mx > 0.f ? kE4M3Max / mx : 0.f;
    char* rd = reinterpret_cast<char*>(dst) + size_t(r) * out_row;
    if (lane == 0) st16(rd, u32x4{__float_as_uint(scale), 0u, 0u, 0u});
    if (lane < npad) st16(rd + 16 + size_t(nvec + lane) * 16, u32x4{0u, 0u, 0u, 0u});
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      const int v = m * 64 + lane;
      if (v < nvec) {
        uint32_t wd[4];
#pragma unroll
        for (int i = 0; i < 4; ++i)
          wd[i] = f32_to_e4m3(f[m][4 * i] * inv) | (f32_to_e4m3(f[m][4 * i + 1] * inv) << 8) |
                  (f32_to_e4m3(f[m][4 * i + 2] * inv) << 16) | (f32_to_e4m3(f[m][4 * i + 3] * inv) << 24);
        st16(rd + 16 + size_t(v) * 16, u32x4{wd[0], wd[1], wd[2], wd[3]});
      }
    }
  }
}

template <typename T, int NVL>
static void launch_gather_nvl(hipStream_t s, const int32_t* idx, const float* w, const void* V, void* y,
                              int64_t ntok, int R, int nvec, const void* target, void* resid) {
  constexpr int U = NVL <= 2 ? 8 : 4;
  dim3 grid(unsigned((ntok + 3) / 4), unsigned((nvec + 64 * NVL - 1) / (64 * NVL)));
  hipLaunchKernelGGL((gather_sum_kernel<T, NVL, U>), grid, dim3(256), 0, s, idx, w,
                     static_cast<const T*>(V), static_cast<T*>(y), ntok, R, nvec, static_cast<const T*>(target),
                     static_cast<T*>(resid));
}

template <typename T>
static void launch_gather_t(hipStream_t s, const int32_t* idx, const float* w, const void* V, void* y,
                            int64_t ntok, int R, int nvec, const void* target, void* resid) {
  // Vectors per lane: enough to cover a row in one column block when the row
  // is at most 256 vectors (4 KB); wider rows use several column blocks.
  const int per_lane = (nvec + 63) / 64;
  if (per_lane <= 1)
    launch_gather_nvl<T, 1>(s, idx, w, V, y, ntok, R, nvec, target, resid);
  else if (per_lane == 2)
    launch_gather_nvl<T, 2>(s, idx, w, V, y, ntok, R, nvec, target, resid);
  else if (per_lane == 3)
    launch_gather_nvl<T, 3>(s, idx, w, V, y, ntok, R, nvec, target, resid);
  else
    launch_gather_nvl<T, 4>(s, idx, w, V, y, ntok, R, nvec, target, resid);
}

template <typename T>
static void launch_gather_fp8_t(hipStream_t s, const int32_t* idx, const float* w, const void* V, void* y,
                                int64_t ntok, int R, int nvec) {
  const dim3 grid(unsigned((ntok + 3) / 4));
  const uint8_t* v8 = static_cast<const uint8_t*>(V);
  T* yo = static_cast<T*>(y);
  const int per_lane = (nvec + 63) / 64;  // nvec <= 256 (rows of <= 4096 codes)
  if (per_lane <= 1)
    hipLaunchKernelGGL((gather_fp8_kernel<T, 1, 8>), grid, dim3(256), 0, s, idx, w, v8, yo, ntok, R, nvec);
  else if (per_lane == 2)
    hipLaunchKernelGGL((gather_fp8_kernel<T, 2, 8>), grid, dim3(256), 0, s, idx, w, v8, yo, ntok, R, nvec);
  else if (per_lane == 3)
    hipLaunchKernelGGL((gather_fp8_kernel<T, 3, 4>), grid, dim3(256), 0, s, idx, w, v8, yo, ntok, R, nvec);
  else
    hipLaunchKernelGGL((gather_fp8_kernel<T, 4, 4>), grid, dim3(256), 0, s, idx, w, v8, yo, ntok, R, nvec);
}

hipError_t launch_gather(hipStream_t s, int dtype, const int32_t* idx, const float* w, const void* V,
                         void* y, int64_t ntok, int R, int d_value, bool fp8_values, const void* target,
                         void* resid) {
  if (fp8_values) {
    if (resid) return hipErrorInvalidValue;
    const int nvec = d_value / 16;
    if (dtype == kBF16)
      launch_gather_fp8_t<bf16_t>(s, idx, w, V, y, ntok, R, nvec);
    else
      launch_gather_fp8_t<float>(s, idx, w, V, y, ntok, R, nvec);
    return hipGetLastError();
  }
  const int elem = dtype == kBF16 ? 2 : 4;
  const int nvec = d_value * elem / 16;
  if (dtype == kBF16)
    launch_gather_t<bf16_t>(s, idx, w, V, y, ntok, R, nvec, target, resid);
  else
    launch_gather_t<float>(s, idx, w, V, y, ntok, R, nvec, target, resid);
  return hipGetLastError();
}

hipError_t launch_quantize_fp8(hipStream_t s, int dtype, const void* src, int64_t rows, int d_value, void* dst) {
  const int nvec = d_value / 16;
  const int per_lane = (nvec + 63) / 64;
  int64_t blocks = (rows + 3) / 4;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) return hipGetLastError();
  uint8_t* d8 = static_cast<uint8_t*>(dst);
#define PKM_QF8(TT, NV) \
  hipLaunchKernelGGL((quantize_fp8_kernel<TT, NV>), dim3(unsigned(blocks)), dim3(256), 0, s, static_cast<const TT*>(src), \
                     rows, nvec, d8)
  if (dtype == kBF16) {
    if (per_lane <= 1) PKM_QF8(bf16_t, 1);
    else if (per_lane == 2) PKM_QF8(bf16_t, 2);
    else if (per_lane == 3) PKM_QF8(bf16_t, 3);
    else PKM_QF8(bf16_t, 4);
  } else {
    if (per_lane <= 1) PKM_QF8(float, 1);
    else if (per_lane == 2) PKM_QF8(float, 2);
    else if (per_lane == 3) PKM_QF8(float, 3);
    else PKM_QF8(float, 4);
  }
#undef PKM_QF8
  return hipGetLastError();
}

}  // namespace pkm
