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
// token slice) the sub-key hits are counted in LDS, one thread per token (a
// token's k slots share few sub-keys, so lanes of different tokens rarely hit
// the same counter at once), and added once per sub-key; every selected row
// stores 1 into its byte of its head's slot map (a plain store: writing the
// same value needs no atomic).  The non-zero bytes of the head maps, and of
// their OR for all heads, are the slots in use.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int kDiagTokens = 256;  // tokens per hit-count block (one per thread)

// Clears up to four buffers (n32[i] 32-bit words each) in one launch.
struct ZeroList {
  uint32_t* p[4];
  int64_t n32[4];
};
__global__ __launch_bounds__(256) void diag_zero_kernel(ZeroList z) {
  for (int b = 0; b < 4; ++b)
    for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < z.n32[b]; i += int64_t(gridDim.x) * 256)
      z.p[b][i] = 0u;
}

__global__ __launch_bounds__(256) void diag_hits_kernel(const int32_t* __restrict__ idx, int64_t ntok, int heads,
                                                        int k, int nk, int nk2, int32_t* __restrict__ hits_c,
                                                        int32_t* __restrict__ hits_cp, uint8_t* __restrict__ maps,
                                                        int64_t map_bytes) {
  extern __shared__ int32_t cnt[];  // [nk + nk2]
  const int hh = blockIdx.y;
  for (int i = threadIdx.x; i < nk + nk2; i += 256) cnt[i] = 0;
  __syncthreads();
  const int64_t t = int64_t(blockIdx.x) * kDiagTokens + threadIdx.x;
  const uint32_t nrows = uint32_t(nk) * uint32_t(nk2);
  uint8_t* map = maps + int64_t(hh) * map_bytes;
  if (t < ntok) {
    const int32_t* it = idx + (t * heads + hh) * k;
    auto count = [&](uint32_t row) {
      if (row < nrows) {  // rows outside the table are not counted
        atomicAdd(&cnt[row / uint32_t(nk2)], 1);
        atomicAdd(&cnt[nk + int(row % uint32_t(nk2))], 1);
        map[row] = 1;
      }
    };
    if ((k & 3) == 0) {  // the token's row ids with 16-byte loads, 4 at a time
      for (int s = 0; s < k; s += 8) {
        const int4 a = *reinterpret_cast<const int4*>(it + s);
        const int4 b = s + 4 < k ? *reinterpret_cast<const int4*>(it + s + 4) : make_int4(-1, -1, -1, -1);
        count(uint32_t(a.x));
        count(uint32_t(a.y));
        count(uint32_t(a.z));
        count(uint32_t(a.w));
        count(uint32_t(b.x));
        count(uint32_t(b.y));
        count(uint32_t(b.z));
        count(uint32_t(b.w));
      }
    } else {
      for (int s = 0; s < k; ++s) count(uint32_t(it[s]));
    }
  }
  __syncthreads();
  for (int i = threadIdx.x; i < nk; i += 256)
    if (cnt[i]) atomicAdd(&hits_c[int64_t(hh) * nk + i], cnt[i]);
  for (int j = threadIdx.x; j < nk2; j += 256)
    if (cnt[nk + j]) atomicAdd(&hits_cp[int64_t(hh) * nk2 + j], cnt[nk + j]);
}

// Non-zero bytes of a 32-bit word of a 0/1 byte map.
__device__ __forceinline__ int bytes_set(uint32_t x) { return __popc(x & 0x01010101u); }

constexpr int kCountWords = 16;  // map words per thread in the count pass

// One pass over the head maps: per head the set bytes of its words (used[1 + h])
// and of their OR over the heads (used[0]); one atomic per block and counter.
__global__ __launch_bounds__(256) void diag_count_kernel(const uint32_t* __restrict__ maps, int64_t map_words,
                                                         int heads, unsigned long long* __restrict__ used) {
  __shared__ int wsum[4];
  const int64_t base = int64_t(blockIdx.x) * 256 * kCountWords + threadIdx.x;
  uint32_t orw[kCountWords];
#pragma unroll
  for (int j = 0; j < kCountWords; ++j) orw[j] = 0u;
  auto block_add = [&](int c, unsigned long long* dst) {
    c = wave_sum_i(c);
    __syncthreads();
    if (lane_id() == 0) wsum[threadIdx.x >> 6] = c;
    __syncthreads();
    if (threadIdx.x == 0) {
      const int tot = wsum[0] + wsum[1] + wsum[2] + wsum[3];
      if (tot) atomicAdd(dst, (unsigned long long)tot);
    }
  };
  for (int hh = 0; hh < heads; ++hh) {
    const uint32_t* m = maps + int64_t(hh) * map_words;
    int c = 0;
#pragma unroll
    for (int j = 0; j < kCountWords; ++j) {
      const int64_t i = base + int64_t(j) * 256;
      const uint32_t x = i < map_words ? m[i] : 0u;
      orw[j] |= x;
      c += bytes_set(x);
    }
    block_add(c, &used[1 + hh]);
  }
  int c = 0;
#pragma unroll
  for (int j = 0; j < kCountWords; ++j) c += bytes_set(orw[j]);
  block_add(c, &used[0]);
}

// Fixed-order sum of the 256 values of a block (tree over LDS); result in sh[0].
__device__ __forceinline__ void block_sum_f64(double* sh) {
  for (int st = 128; st > 0; st >>= 1) {
    __syncthreads();
    if (threadIdx.x < st) sh[threadIdx.x] += sh[threadIdx.x + st];
  }
  __syncthreads();
}

// Entropy of every (t, h) item (n = T*h): eight lanes per item, lane j taking
// weights 4j.. (16-byte loads when k is a multiple of 4), a fixed xor-tree sum
// over the eight; per-block fp64 partial sums of the 32 items of the block.
__global__ __launch_bounds__(256) void diag_entropy_kernel(const float* __restrict__ w, int64_t n, int k,
                                                           float* __restrict__ ent, double* __restrict__ part) {
  __shared__ double sh[256];
  const int sub = threadIdx.x & 7;
  double acc = 0.0;  // this lane group's items, in a fixed order
  // every lane of the block takes the same number of steps (the test is on the
  // block's first item), so the shuffles below always see the whole wave
  for (int64_t i = int64_t(blockIdx.x) * 32 + (threadIdx.x >> 3); i - (threadIdx.x >> 3) < n;
       i += int64_t(gridDim.x) * 32) {
    float e = 0.f;
    if (i < n) {
      const float* wi = w + i * k;
      if ((k & 3) == 0) {
        for (int s = 4 * sub; s < k; s += 32) {
          const f32x4 x = *reinterpret_cast<const f32x4*>(wi + s);
#pragma unroll
          for (int q = 0; q < 4; ++q)
            if (x[q] > 0.f) e -= x[q] * logf(x[q]);
        }
      } else {
        for (int s = sub; s < k; s += 8) {
          const float x = wi[s];
          if (x > 0.f) e -= x * logf(x);
        }
      }
    }
    e += __shfl_xor(e, 1, 64);
    e += __shfl_xor(e, 2, 64);
    e += __shfl_xor(e, 4, 64);
    if (sub == 0 && i < n && ent) ent[i] = e;
    if (sub == 0 && i < n) acc += double(e);
  }
  sh[threadIdx.x] = acc;
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
// entropy launch: groups of 32 items, at most 1024 blocks (one fp64 partial each)
inline int64_t entropy_blocks(int64_t n) {
  const int64_t b = (n + 31) / 32;
  return b < 1 ? 1 : b > 1024 ? 1024 : b;
}
inline int64_t map_bytes_of(int64_t nrows) { return (nrows + 255) / 256 * 256; }  // whole 32-bit words, aligned

}  // namespace

size_t diagnostics_ws_bytes(int64_t ntok, int heads, int64_t nrows) {
  return al256(size_t(heads) * size_t(map_bytes_of(nrows))) + al256(size_t(entropy_blocks(ntok * heads)) * 8);
}

hipError_t launch_diagnostics(hipStream_t s, const int32_t* idx, const float* w, int64_t ntok, int heads, int k,
                              int nk, int nk2, int32_t* hits_c, int32_t* hits_cp, int64_t* used, float* entropy,
                              double* entropy_sum, void* ws) {
  const int64_t nrows = int64_t(nk) * nk2;
  const int64_t mb = map_bytes_of(nrows);
  uint8_t* maps = static_cast<uint8_t*>(ws);
  double* part = reinterpret_cast<double*>(static_cast<char*>(ws) + al256(size_t(heads) * size_t(mb)));
  ZeroList z;
  z.p[0] = reinterpret_cast<uint32_t*>(hits_c);
  z.n32[0] = int64_t(heads) * nk;
  z.p[1] = reinterpret_cast<uint32_t*>(hits_cp);
  z.n32[1] = int64_t(heads) * nk2;
  z.p[2] = reinterpret_cast<uint32_t*>(used);
  z.n32[2] = 2 * int64_t(1 + heads);
  z.p[3] = reinterpret_cast<uint32_t*>(maps);
  z.n32[3] = int64_t(heads) * mb / 4;
  int64_t zb = (z.n32[3] + 255) / 256;
  if (zb > 2048) zb = 2048;
  if (zb < 1) zb = 1;
  hipLaunchKernelGGL(diag_zero_kernel, dim3(unsigned(zb)), dim3(256), 0, s, z);
  if (ntok == 0) {
    if (entropy_sum) {
      ZeroList z2 = {};
      z2.p[0] = reinterpret_cast<uint32_t*>(entropy_sum);
      z2.n32[0] = 2;
      for (int b = 1; b < 4; ++b) z2.p[b] = nullptr;
      hipLaunchKernelGGL(diag_zero_kernel, dim3(1), dim3(256), 0, s, z2);
    }
    return hipGetLastError();
  }
  const dim3 gh(unsigned((ntok + kDiagTokens - 1) / kDiagTokens), unsigned(heads));
  hipLaunchKernelGGL(diag_hits_kernel, gh, dim3(256), size_t(nk + nk2) * 4, s, idx, ntok, heads, k, nk, nk2, hits_c,
                     hits_cp, maps, mb);
  const int64_t words = mb / 4;
  const int64_t cb = (words + 256 * kCountWords - 1) / (256 * kCountWords);
  hipLaunchKernelGGL(diag_count_kernel, dim3(unsigned(cb)), dim3(256), 0, s, reinterpret_cast<const uint32_t*>(maps),
                     words, heads, reinterpret_cast<unsigned long long*>(used));
  const int64_t n = ntok * heads;
  const int64_t nblk = entropy_blocks(n);
  hipLaunchKernelGGL(diag_entropy_kernel, dim3(unsigned(nblk)), dim3(256), 0, s, w, n, k, entropy, part);
  if (entropy_sum) hipLaunchKernelGGL(diag_sum_kernel, dim3(1), dim3(256), 0, s, part, nblk, entropy_sum);
  return hipGetLastError();
}

}  // namespace pkm
