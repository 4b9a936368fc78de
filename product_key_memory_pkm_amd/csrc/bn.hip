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
// block order by one thread per feature: no atomics, bit-identical across runs.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

__global__ __launch_bounds__(256) void bn_partials_kernel(const float* __restrict__ q_pre, int64_t ntok, int F,
                                                          double* __restrict__ part) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int64_t r1 = r0 + kBnRows < ntok ? r0 + kBnRows : ntok;
  double s = 0.0, ss = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const double v = q_pre[r * F + f];
    s += v;
    ss += v * v;
  }
  part[(int64_t(blockIdx.y) * 2 + 0) * F + f] = s;
  part[(int64_t(blockIdx.y) * 2 + 1) * F + f] = ss;
}

__global__ __launch_bounds__(256) void bn_finalize_kernel(const double* __restrict__ part, int nblk, int64_t ntok,
                                                          int F, float eps, float* __restrict__ mean,
                                                          float* __restrict__ rstd) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  double s = 0.0, ss = 0.0;
  for (int b = 0; b < nblk; ++b) {
    s += part[(int64_t(b) * 2 + 0) * F + f];
    ss += part[(int64_t(b) * 2 + 1) * F + f];
  }
  const double m = s / double(ntok);
  double var = ss / double(ntok) - m * m;
  if (var < 0.0) var = 0.0;
  mean[f] = float(m);
  rstd[f] = float(1.0 / sqrt(var + double(eps)));
}

template <typename T>
__global__ __launch_bounds__(256) void bn_apply_kernel(const float* __restrict__ q_pre, int64_t n4, int F,
                                                       const float* __restrict__ mean,
                                                       const float* __restrict__ rstd,
                                                       const float* __restrict__ gamma,
                                                       const float* __restrict__ beta, int bn, T* __restrict__ q) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    const float4 v = reinterpret_cast<const float4*>(q_pre)[i];
    const int f = int((i * 4) % F);
    float o[4] = {v.x, v.y, v.z, v.w};
    if (bn) {
#pragma unroll
      for (int e = 0; e < 4; ++e) o[e] = gamma[f + e] * ((o[e] - mean[f + e]) * rstd[f + e]) + beta[f + e];
    }
#pragma unroll
    for (int e = 0; e < 4; ++e) q[i * 4 + e] = to_storage<T>(o[e]);
  }
}

__global__ __launch_bounds__(256) void bn_bwd_partials_kernel(const float* __restrict__ dq,
                                                              const float* __restrict__ q_pre,
                                                              const float* __restrict__ mean,
                                                              const float* __restrict__ rstd, int64_t ntok, int F,
                                                              double* __restrict__ part) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  const int64_t r0 = int64_t(blockIdx.y) * kBnRows;
  const int64_t r1 = r0 + kBnRows < ntok ? r0 + kBnRows : ntok;
  const float mu = mean[f], rs = rstd[f];
  double s = 0.0, sx = 0.0;
  for (int64_t r = r0; r < r1; ++r) {
    const float g = dq[r * F + f];
    const float xh = (q_pre[r * F + f] - mu) * rs;
    s += double(g);
    sx += double(g) * double(xh);
  }
  part[(int64_t(blockIdx.y) * 2 + 0) * F + f] = s;
  part[(int64_t(blockIdx.y) * 2 + 1) * F + f] = sx;
}

__global__ __launch_bounds__(256) void bn_bwd_finalize_kernel(const double* __restrict__ part, int nblk, int F,
                                                              float* __restrict__ dgamma,
                                                              float* __restrict__ dbeta) {
  const int f = blockIdx.x * 256 + threadIdx.x;
  if (f >= F) return;
  double s = 0.0, sx = 0.0;
  for (int b = 0; b < nblk; ++b) {
    s += part[(int64_t(b) * 2 + 0) * F + f];
    sx += part[(int64_t(b) * 2 + 1) * F + f];
  }
  dbeta[f] = float(s);
  dgamma[f] = float(sx);
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
                                                           int bn, T* __restrict__ out_rm, T* __restrict__ out_tr,
                                                           int64_t ld_tr, int64_t rows_pad) {
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
      out_rm[r * F + f] = to_storage<T>(v);
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
  dim3 grid(unsigned((F + 255) / 256), unsigned((ntok + kBnRows - 1) / kBnRows));
  hipLaunchKernelGGL(bn_partials_kernel, grid, dim3(256), 0, s, q_pre, ntok, F, part);
  return hipGetLastError();
}

hipError_t launch_bn_finalize(hipStream_t s, const double* part, int nblk, int64_t ntok, int F, float eps,
                              float* mean, float* rstd) {
  hipLaunchKernelGGL(bn_finalize_kernel, dim3(unsigned((F + 255) / 256)), dim3(256), 0, s, part, nblk, ntok, F,
                     eps, mean, rstd);
  return hipGetLastError();
}

hipError_t launch_bn_apply(hipStream_t s, int dtype, const float* q_pre, int64_t ntok, int F, const float* mean,
                           const float* rstd, const float* gamma, const float* beta, void* q) {
  const int64_t n4 = ntok * F / 4;  // F % 4 == 0
  const int bn = mean != nullptr;
  if (dtype == kBF16)
    hipLaunchKernelGGL(bn_apply_kernel<bf16_t>, dim3(grid1d(n4)), dim3(256), 0, s, q_pre, n4, F, mean, rstd, gamma,
                       beta, bn, static_cast<bf16_t*>(q));
  else
    hipLaunchKernelGGL(bn_apply_kernel<float>, dim3(grid1d(n4)), dim3(256), 0, s, q_pre, n4, F, mean, rstd, gamma,
                       beta, bn, static_cast<float*>(q));
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
  hipLaunchKernelGGL(bn_bwd_finalize_kernel, dim3(unsigned((F + 255) / 256)), dim3(256), 0, s, part, nblk, F,
                     dgamma, dbeta);
  return hipGetLastError();
}

hipError_t launch_bn_bwd_apply(hipStream_t s, int dtype, const float* dq, const float* q_pre, const float* mean,
                               const float* rstd, const float* gamma, const float* dgamma, const float* dbeta,
                               int64_t ntok, int F, bool bn, void* out_rm, void* out_tr, int64_t ld_tr) {
  dim3 grid(unsigned((F + 63) / 64), unsigned((ld_tr + 63) / 64));
  if (dtype == kBF16)
    hipLaunchKernelGGL(bn_bwd_apply_kernel<bf16_t>, grid, dim3(256), 0, s, dq, q_pre, mean, rstd, gamma, dgamma,
                       dbeta, ntok, F, int(bn), static_cast<bf16_t*>(out_rm), static_cast<bf16_t*>(out_tr), ld_tr,
                       ld_tr);
  else
    hipLaunchKernelGGL(bn_bwd_apply_kernel<float>, grid, dim3(256), 0, s, dq, q_pre, mean, rstd, gamma, dgamma,
                       dbeta, ntok, F, int(bn), static_cast<float*>(out_rm), static_cast<float*>(out_tr), ld_tr,
                       ld_tr);
  return hipGetLastError();
}

}  // namespace pkm
