// Monitoring signals of one batch's selection ("Meta AI 可扩展内存层",
// section 11.2: the codebook hit distribution, the hit count of every sub-key
// and the candidate softmax entropy are the signals to watch; section 9.3:
// per-sub-key hit counts and gradient density; product-key paper summary, key
// results: memory usage, the share of slots in use).
//
//   hits_c[h, i]  = #{(t, s): idx[t,h,s] / |C'| == i}
//   hits_cp[h, j] = #{(t, s): idx[t,h,s] % |C'| == j}
//   used[0]       = #distinct idx over the batch, used[1 + h] = the same for head h
//   entropy[t, h] = -sum_s w log w,  entropy_sum = sum over (t, h), fp64 in a fixed order
//
// Counts are integers (atomics give exact, order-free results): per (head,
// token slice) the sub-key hits are counted in LDS and added once per sub-key;
// every selected row sets its bit in an all-heads and a per-head slot bitmap,
// whose popcounts are the slots in use.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int kDiagTokens = 256;  // tokens per hit-count block

__global__ __launch_bounds__(256) void diag_hits_kernel(const int32_t* __restrict__ idx, int64_t ntok, int heads,
                                                        int k, int nk, int nk2, int32_t* __restrict__ hits_c,
                                                        int32_t* __restrict__ hits_cp, uint32_t* __restrict__ bitmaps,
                                                        int64_t bm_words) {
  extern __shared__ int32_t cnt[];  // [nk + nk2]
  const int hh = blockIdx.y;
  for (int i = threadIdx.x; i < nk + nk2; i += 256) cnt[i] = 0;
  __syncthreads();
  const int64_t t0 = int64_t(blockIdx.x) * kDiagTokens;
  const int64_t t1 = t0 + kDiagTokens < ntok ? t0 + kDiagTokens : ntok;
  const int64_t n = (t1 - t0) * k;
  const uint32_t nrows = uint32_t(nk) * uint32_t(nk2);
  uint32_t* bm_all = bitmaps;
  uint32_t* bm_h = bitmaps + int64_t(1 + hh) * bm_words;
  for (int64_t e = threadIdx.x; e < n; e += 256) {
    const int64_t t = t0 + e / k;
    const int s = int(e % k);
    const uint32_t row = uint32_t(idx[(t * heads + hh) * k + s]);
    if (row < nrows) {  // rows outside the table are not counted
      atomicAdd(&cnt[row / uint32_t(nk2)], 1);
      atomicAdd(&cnt[nk + int(row % uint32_t(nk2))], 1);
      atomicOr(&bm_all[row >> 5], 1u << (row & 31));
      atomicOr(&bm_h[row >> 5], 1u << (row & 31));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nk; i += 256)
    if (cnt[i]) atomicAdd(&hits_c[int64_t(hh) * nk + i], cnt[i]);
  for (int j = threadIdx.x; j < nk2; j += 256)
    if (cnt[nk + j]) atomicAdd(&hits_cp[int64_t(hh) * nk2 + j], cnt[nk + j]);
}

// used[b] += set bits of bitmap b (grid.y = bitmap)
__global__ __launch_bounds__(256) void diag_popc_kernel(const uint32_t* __restrict__ bitmaps, int64_t bm_words,
                                                        unsigned long long* __restrict__ used) {
  const uint32_t* bm = bitmaps + int64_t(blockIdx.y) * bm_words;
  int c = 0;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < bm_words; i += int64_t(gridDim.x) * 256)
    c += __popc(bm[i]);
  c = wave_sum_i(c);
  if (lane_id() == 0 && c) atomicAdd(&used[blockIdx.y], (unsigned long long)c);
}

// Fixed-order sum of the 256 values of a block (tree over LDS); result in sh[0].
__device__ __forceinline__ void block_sum_f64(double* sh) {
  for (int st = 128; st > 0; st >>= 1) {
    __syncthreads();
    if (threadIdx.x < st) sh[threadIdx.x] += sh[threadIdx.x + st];
  }
  __syncthreads();
}

// entropy of every (t, h) item (n = T*h) and per-block fp64 partial sums
__global__ __launch_bounds__(256) void diag_entropy_kernel(const float* __restrict__ w, int64_t n, int k,
                                                           float* __restrict__ ent, double* __restrict__ part) {
  __shared__ double sh[256];
  const int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x;
  float e = 0.f;
  if (i < n) {
    const float* wi = w + i * k;
    for (int s = 0; s < k; ++s) {
      const float x = wi[s];
      if (x > 0.f) e -= x * logf(x);
    }
    if (ent) ent[i] = e;
  }
  sh[threadIdx.x] = double(e);
  block_sum_f64(sh);
  if (threadIdx.x == 0) part[blockIdx.x] = sh[0];
}

__global__ __launch_bounds__(256) void diag_sum_kernel(const double* __restrict__ part, int64_t nblk,
                                                       double* __restrict__ out) {
  __shared__ double sh[256];
  double s = 0.0;
  for (int64_t b = threadIdx.x; b < nblk; b += 256) s += part[b];
  sh[threadIdx.x] = s;
  block_sum_f64(sh);
  if (threadIdx.x == 0) *out = sh[0];
}

inline size_t al256(size_t b) { return (b + 255) / 256 * 256; }

}  // namespace

size_t diagnostics_ws_bytes(int64_t ntok, int heads, int64_t nrows) {
  const int64_t words = (nrows + 31) / 32;
  const int64_t nblk = (ntok * heads + 255) / 256;
  return al256(size_t(1 + heads) * size_t(words) * 4) + al256(size_t(nblk > 0 ? nblk : 1) * 8);
}

hipError_t launch_diagnostics(hipStream_t s, const int32_t* idx, const float* w, int64_t ntok, int heads, int k,
                              int nk, int nk2, int32_t* hits_c, int32_t* hits_cp, int64_t* used, float* entropy,
                              double* entropy_sum, void* ws) {
  const int64_t nrows = int64_t(nk) * nk2;
  const int64_t words = (nrows + 31) / 32;
  uint32_t* bitmaps = static_cast<uint32_t*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + al256(size_t(1 + heads) * size_t(words) * 4));
  hipError_t e;
  // every fill writes zero bits (int32 / int64 / uint32 zeros)
  if ((e = launch_fill_f32(s, reinterpret_cast<float*>(hits_c), int64_t(heads) * nk, 0.f)) != hipSuccess) return e;
  if ((e = launch_fill_f32(s, reinterpret_cast<float*>(hits_cp), int64_t(heads) * nk2, 0.f)) != hipSuccess) return e;
  if ((e = launch_fill_f32(s, reinterpret_cast<float*>(used), 2 * int64_t(1 + heads), 0.f)) != hipSuccess) return e;
  if ((e = launch_fill_f32(s, reinterpret_cast<float*>(bitmaps), int64_t(1 + heads) * words, 0.f)) != hipSuccess)
    return e;
  if (entropy_sum && (e = launch_fill_f32(s, reinterpret_cast<float*>(entropy_sum), 2, 0.f)) != hipSuccess) return e;
  if (ntok == 0) return hipGetLastError();
  const dim3 gh(unsigned((ntok + kDiagTokens - 1) / kDiagTokens), unsigned(heads));
  hipLaunchKernelGGL(diag_hits_kernel, gh, dim3(256), size_t(nk + nk2) * 4, s, idx, ntok, heads, k, nk, nk2, hits_c,
                     hits_cp, bitmaps, words);
  int64_t pb = (words + 255) / 256;
  if (pb > 1024) pb = 1024;
  hipLaunchKernelGGL(diag_popc_kernel, dim3(unsigned(pb), unsigned(1 + heads)), dim3(256), 0, s, bitmaps, words,
                     reinterpret_cast<unsigned long long*>(used));
  const int64_t n = ntok * heads;
  const int64_t nblk = (n + 255) / 256;
  hipLaunchKernelGGL(diag_entropy_kernel, dim3(unsigned(nblk)), dim3(256), 0, s, w, n, k, entropy, part);
  if (entropy_sum) hipLaunchKernelGGL(diag_sum_kernel, dim3(1), dim3(256), 0, s, part, nblk, entropy_sum);
  return hipGetLastError();
}

}  // namespace pkm
