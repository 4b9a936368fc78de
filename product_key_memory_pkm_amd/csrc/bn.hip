// Step a2 and the BatchNorm part of a10: batch-statistics BatchNorm on the
// query features (product-key paper summary, key results: BatchNorm in the
// query network raises memory usage).
//
//   mean_f = (1/T) sum_t q_pre[t,f];  var_f = (1/T) sum_t q_pre[t,f]^2 - mean_f^2
//   q[t,f] = gamma_f (q_pre[t,f] - mean_f) / sqrt(var_f + eps) + beta_f
//   backward: dbeta_f = sum_t dq, dgamma_f = sum_t dq xhat,
//             dq_pre = gamma_f rstd_f (dq - dbeta_f/T - xhat dgamma_f/T)
//
// Column sums are taken in fp64 over fixed blocks of 256 rows, then combined in
// a fixed order (four strided groups of blocks, added group by group): no
// atomics, bit-identical across runs.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

// Thread (ty, tx) of a block sums features 4*tx.. of the block's 256-feature
// slice over rows ty, ty+4, ... of its row block (fp64, four features at
// once); the four row groups are then added in a fixed order through LDS.
__device__ __forceinline__ void bn_combine_store(double (*acc)[4], double* __restrict__ part, int F, int f4) {
  __shared__ double red[4][2][4][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
#pragma unroll
  for (int a = 0; a < 2; ++a)
#pragma unroll
    for (int e = 0; e < 4; ++e) red[ty][a][e][tx] = acc[a][e];
  __syncthreads();
  if (ty == 0 && f4 < F) {
#pragma unroll
    for (int a = 0; a < 2; ++a)
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double v = ((red[0][a][e][tx] + red[1][a][e][tx]) + red[2][a][e][tx]) + red[3][a][e][tx];
        part[(int64_t(blockIdx.y) * 2 + a) * F + f4 + e] = v;
      }
  }
}

__global__ __launch_bounds__(256) void bn_partials_kernel(const float* __restrict__ q_pre, int64_t ntok, int F,
                                                          double* __restrict__ part) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int f4 = (blockIdx.x * 64 + tx) * 4;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int64_t r1 = r0 + kBnRows < ntok ? r0 + kBnRows : ntok;
  double acc[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  if (f4 < F) {
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      const f32x4 v = *reinterpret_cast<const f32x4*>(q_pre + r * F + f4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const double d = v[e];
        acc[0][e] += d;
        acc[1][e] += d * d;
      }
    }
  }
  bn_combine_store(acc, part, F, f4);
}

// Thread (ty, tx) of a block adds partial blocks ty, ty+4, ... of feature
// 64 * blockIdx.x + tx; the four row-group sums are combined in a fixed order.
__device__ __forceinline__ void bn_sum_partials(const double* __restrict__ part, int nblk, int F, double* out2) {
  __shared__ double red[4][2][64];
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int f = blockIdx.x * 64 + tx;
  double a = 0.0, b = 0.0;
  if (f < F)
    for (int k = ty; k < nblk; k += 4) {
      a += part[(int64_t(k) * 2 + 0) * F + f];
      b += part[(int64_t(k) * 2 + 1) * F + f];
    }
  red[ty][0][tx] = a;
  red[ty][1][tx] = b;
  __syncthreads();
  out2[0] = ((red[0][0][tx] + red[1][0][tx]) + red[2][0][tx]) + red[3][0][tx];
  out2[1] = ((red[0][1][tx] + red[1][1][tx]) + red[2][1][tx]) + red[3][1][tx];
}

__global__ __launch_bounds__(256) void bn_finalize_kernel(const double* __restrict__ part, int nblk, int64_t ntok,
                                                          int F, float eps, float* __restrict__ mean,
                                                          float* __restrict__ rstd) {
  double sums[2];
  bn_sum_partials(part, nblk, F, sums);
  const int f = blockIdx.x * 64 + (threadIdx.x & 63);
  if (threadIdx.x >= 64 || f >= F) return;
  const double m = sums[0] / double(ntok);
  double var = sums[1] / double(ntok) - m * m;
  if (var < 0.0) var = 0.0;
  mean[f] = float(m);
  rstd[f] = float(1.0 / sqrt(var + double(eps)));
}

// Thread tx of a block normalises features 4*tx.. of a 1024-feature slice for
// kApplyRows consecutive rows (no per-element index arithmetic).
constexpr int kApplyRows = 8;

template <typename T>
__device__ __forceinline__ void store4(T* p, const float* o);
template <>
__device__ __forceinline__ void store4<bf16_t>(bf16_t* p, const float* o) {
  const uint32_t lo = uint32_t(f32_to_bf16(o[0])) | (uint32_t(f32_to_bf16(o[1])) << 16);
  const uint32_t hi = uint32_t(f32_to_bf16(o[2])) | (uint32_t(f32_to_bf16(o[3])) << 16);
  *reinterpret_cast<u32x2*>(p) = u32x2{lo, hi};
}
template <>
__device__ __forceinline__ void store4<float>(float* p, const float* o) {
  *reinterpret_cast<f32x4*>(p) = f32x4{o[0], o[1], o[2], o[3]};
}

template <typename T>
__global__ __launch_bounds__(256) void bn_apply_kernel(const float* __restrict__ q_pre, int64_t ntok, int F,
                                                       const float* __restrict__ mean,
                                                       const float* __restrict__ rstd,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, int bn, T* __restrict__ q) {
  const int f4 = (blockIdx.x * 256 + threadIdx.x) * 4;
  if (f4 >= F) return;
  float mu[4] = {0.f, 0.f, 0.f, 0.f}, rs[4] = {1.f, 1.f, 1.f, 1.f}, ga[4] = {1.f, 1.f, 1.f, 1.f},
        be[4] = {0.f, 0.f, 0.f, 0.f};
  if (bn) {
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mu[e] = mean[f4 + e];
      rs[e] = rstd[f4 + e];
      ga[e] = gamma[f4 + e];
      be[e] = beta[f4 + e];
    }
  }
  const int64_t r0 = int64_t(blockIdx.y) * kApplyRows;
  const int64_t r1 = r0 + kApplyRows < ntok ? r0 + kApplyRows : ntok;
  for (int64_t r = r0; r < r1; ++r) {
    const f32x4 v = *reinterpret_cast<const f32x4*>(q_pre + r * F + f4);
    float o[4] = {v.x, v.y, v.z, v.w};
    if (bn) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = ga[e] * ((o[e] - mu[e]) * rs[e]) + be[e];
    }
    store4<T>(q + r * F + f4, o);
  }
}

__global__ __launch_bounds__(256) void bn_bwd_partials_kernel(const float* __restrict__ dq,
                                                              const float* __restrict__ q_pre,
                                                              const float* __restrict__ mean,
                                                              const float* __restrict__ rstd, int64_t ntok, int F,
                                                              double* __restrict__ part) {
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int f4 = (blockIdx.x * 64 + tx) * 4;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int64_t r1 = r0 + kBnRows < ntok ? r0 + kBnRows : ntok;
  double acc[2][4] = {{0.0, 0.0, 0.0, 0.0}, {0.0, 0.0, 0.0, 0.0}};
  if (f4 < F) {
    float mu[4], rs[4];
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      mu[e] = mean[f4 + e];
      rs[e] = rstd[f4 + e];
    }
    for (int64_t r = r0 + ty; r < r1; r += 4) {
      const f32x4 g = *reinterpret_cast<const f32x4*>(dq + r * F + f4);
      const f32x4 x = *reinterpret_cast<const f32x4*>(q_pre + r * F + f4);
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const float xh = (x[e] - mu[e]) * rs[e];
        acc[0][e] += double(g[e]);
        acc[1][e] += double(g[e]) * double(xh);
      }
    }
  }
  bn_combine_store(acc, part, F, f4);
}

__global__ __launch_bounds__(256) void bn_bwd_finalize_kernel(const double* __restrict__ part, int nblk, int F,
                                                              float* __restrict__ dgamma,
                                                              float* __restrict__ dbeta) {
  double sums[2];
  bn_sum_partials(part, nblk, F, sums);
  const int f = blockIdx.x * 64 + (threadIdx.x & 63);
  if (threadIdx.x >= 64 || f >= F) return;
  dbeta[f] = float(sums[0]);
  dgamma[f] = float(sums[1]);
}

// 64 x 64 tiles: dq_pre written row-major and, through LDS, transposed.
template <typename T>
__global__ __launch_bounds__(256) void bn_bwd_apply_kernel(const float* __restrict__ dq,
                                                           const float* __restrict__ q_pre,
                                                           const float* __restrict__ mean,
                                                           const float* __restrict__ rstd,
                                                           const float* __restrict__ gamma,
                                                           const float* __restrict__ dgamma,
                                                           const float* __restrict__ dbeta, int64_t ntok, int F,
                                                           int bn, T* __restrict__ out_rm, int64_t ld_rm,
                                                           T* __restrict__ out_tr, int64_t ld_tr, int64_t rows_pad) {
  __shared__ float tile[64][65];
  const int64_t r0 = int64_t(blockIdx.y) * 64;
  const int f0 = blockIdx.x * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  const int f = f0 + tx;
  float a = 0.f, c1 = 0.f, c2 = 0.f, mu = 0.f, rs = 1.f;
  if (f < F && bn) {
    const float invT = 1.0f / float(ntok);
    mu = mean[f];
    rs = rstd[f];
    a = gamma[f] * rs;
    c1 = dbeta[f] * invT;
    c2 = dgamma[f] * invT;
  }
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i;
    float v = 0.f;
    if (r < ntok && f < F) {
      const float g = dq[r * F + f];
      if (bn) {
        const float xh = (q_pre[r * F + f] - mu) * rs;
        v = a * (g - c1 - xh * c2);
      } else {
        v = g;
      }
      out_rm[r * ld_rm + f] = to_storage<T>(v);
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int ff = f0 + i;
    const int64_t r = r0 + tx;
    if (ff < F && r < rows_pad) out_tr[int64_t(ff) * ld_tr + r] = to_storage<T>(tile[tx][i]);
  }
}

inline unsigned grid1d(int64_t n, int64_t cap = 8192) {
  int64_t b = (n + 255) / 256;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return unsigned(b);
}

}  // namespace

hipError_t launch_bn_partials(hipStream_t s, const float* q_pre, int64_t ntok, int F, double* part) {
  dim3 grid(unsigned((F + 255) / 256), unsigned((ntok + kBnRows - 1) / kBnRows));  // F % 4 == 0
  hipLaunchKernelGGL(bn_partials_kernel, grid, dim3(256), 0, s, q_pre, ntok, F, part);
  return hipGetLastError();
}

hipError_t launch_bn_finalize(hipStream_t s, const double* part, int nblk, int64_t ntok, int F, float eps,
                              float* mean, float* rstd) {
  hipLaunchKernelGGL(bn_finalize_kernel, dim3(unsigned((F + 63) / 64)), dim3(256), 0, s, part, nblk, ntok, F,
                     eps, mean, rstd);
  return hipGetLastError();
}

hipError_t launch_bn_apply(hipStream_t s, int dtype, const float* q_pre, int64_t ntok, int F, const float* mean,
                           const float* rstd, const float* gamma, const float* beta, void* q) {
  if (ntok == 0) return hipSuccess;
  const int bn = mean != nullptr;
  const dim3 grid(unsigned((F / 4 + 255) / 256), unsigned((ntok + kApplyRows - 1) / kApplyRows));  // F % 4 == 0
  if (dtype == kBF16)
    hipLaunchKernelGGL(bn_apply_kernel<bf16_t>, grid, dim3(256), 0, s, q_pre, ntok, F, mean, rstd, gamma, beta, bn,
                       static_cast<bf16_t*>(q));
  else
    hipLaunchKernelGGL(bn_apply_kernel<float>, grid, dim3(256), 0, s, q_pre, ntok, F, mean, rstd, gamma, beta, bn,
                       static_cast<float*>(q));
  return hipGetLastError();
}

hipError_t launch_bn_bwd_partials(hipStream_t s, const float* dq, const float* q_pre, const float* mean,
                                  const float* rstd, int64_t ntok, int F, double* part) {
  dim3 grid(unsigned((F + 255) / 256), unsigned((ntok + kBnRows - 1) / kBnRows));
  hipLaunchKernelGGL(bn_bwd_partials_kernel, grid, dim3(256), 0, s, dq, q_pre, mean, rstd, ntok, F, part);
  return hipGetLastError();
}

hipError_t launch_bn_bwd_finalize(hipStream_t s, const double* part, int nblk, int F, const float* gamma,
                                  float* dgamma, float* dbeta, float* coef) {
  (void)gamma;
  (void)coef;
  hipLaunchKernelGGL(bn_bwd_finalize_kernel, dim3(unsigned((F + 63) / 64)), dim3(256), 0, s, part, nblk, F,
                     dgamma, dbeta);
  return hipGetLastError();
}

hipError_t launch_bn_bwd_apply(hipStream_t s, int dtype, const float* dq, const float* q_pre, const float* mean,
                               const float* rstd, const float* gamma, const float* dgamma, const float* dbeta,
                               int64_t ntok, int F, bool bn, void* out_rm, int64_t ld_rm, void* out_tr, int64_t ld_tr,
                               int64_t rows_pad) {
  dim3 grid(unsigned((F + 63) / 64), unsigned((rows_pad + 63) / 64));
  if (dtype == kBF16)
    hipLaunchKernelGGL(bn_bwd_apply_kernel<bf16_t>, grid, dim3(256), 0, s, dq, q_pre, mean, rstd, gamma, dgamma,
                       dbeta, ntok, F, int(bn), static_cast<bf16_t*>(out_rm), ld_rm, static_cast<bf16_t*>(out_tr),
                       ld_tr, rows_pad);
  else
    hipLaunchKernelGGL(bn_bwd_apply_kernel<float>, grid, dim3(256), 0, s, dq, q_pre, mean, rstd, gamma, dgamma,
                       dbeta, ntok, F, int(bn), static_cast<float*>(out_rm), ld_rm, static_cast<float*>(out_tr),
                       ld_tr, rows_pad);
  return hipGetLastError();
}

}  // namespace pkm
