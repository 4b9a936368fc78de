// Step a5: k x k candidate merge, top-k of the candidates, softmax.
//
// For the sorted per-half lists (I1, s1) and (I2, s2) of one (token, head):
//   candidate (a, b): score s1[a] + s2[b], row I1[a] * |C'| + I2[b]
//   keep the k best by (score desc, row asc); w = softmax(score / tau).
// ("Meta AI 可扩展内存层", sections 4.3 and 4.5: Cartesian candidates, full-key
// score as the sum of the half scores, row by offset; product-key paper
// summary, method details: the candidate set is searched for the k best keys.)
//
// Only pairs with (a+1)(b+1) <= k can be among the k best: every (a', b') with
// a' <= a, b' <= b scores at least as much and, on an equal score, has the
// lower row (the per-half lists are ordered by score, then index).  For k = 32
// that leaves 119 of the 1024 pairs.  (Exact for the sums as real numbers; an
// equality that only fp32 rounding creates between sums of different halves
// can keep another of the equal-scoring rows than an exhaustive fp32 merge.)  One wave per (token, head): each lane
// builds up to two candidates, the k-th largest 64-bit key (score key, ~row)
// is found by bisection with ballots, the k winners are compacted and sorted
// with a 32-lane bitonic network, and the softmax runs on the sorted lanes.
#include "common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkm {

namespace {

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Bitonic sort, descending, of one uint64 per lane within aligned groups of 32
// lanes (every exchange stays inside 32 lanes: DPP or ds_swizzle).
__device__ __forceinline__ uint64_t sort32_desc_u64(uint64_t v) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 32; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const uint64_t o = xor_lane_u64(v, stride);
      const bool take_max = ((lane & stride) == 0) == ((lane & size) == 0 || size == 32);
      const bool gt = v > o;
      v = (gt == take_max) ? v : o;
    }
  }
  return v;
}

constexpr int kWavesPerBlock = 4;

__global__ __launch_bounds__(256) void merge_softmax_kernel(const int32_t* __restrict__ sub_idx,
                                                            const float* __restrict__ sub_score,
                                                            int64_t nitems, int k, int nk2, float inv_tau,
                                                            int32_t* __restrict__ idx, float* __restrict__ w,
                                                            float* __restrict__ score, int64_t group_items,
                                                            int64_t group_rows, int64_t group_count) {
  __shared__ uint16_t pairs[128];
  __shared__ int npairs;
  __shared__ uint64_t scratch[kWavesPerBlock][64];
  if (threadIdx.x == 0) {
    int c = 0;
    for (int a = 0; a < k; ++a) {
      const int nb = k / (a + 1);
      for (int b = 0; b < nb; ++b) pairs[c++] = uint16_t(a | (b << 8));
    }
    npairs = c;
  }
  __syncthreads();
  const int P = npairs;
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  uint16_t pr0 = lane < P ? pairs[lane] : 0;
  uint16_t pr1 = lane + 64 < P ? pairs[lane + 64] : 0;
  const int a0 = pr0 & 0xFF, b0 = pr0 >> 8, a1 = pr1 & 0xFF, b1 = pr1 >> 8;
  uint64_t* scr = scratch[wave];

  for (int64_t it = int64_t(blockIdx.x) * kWavesPerBlock + wave; it < nitems;
       it += int64_t(gridDim.x) * kWavesPerBlock) {
    const int32_t* si = sub_idx + it * 2 * k;
    const float* ss = sub_score + it * 2 * k;
    const float v1 = lane < k ? ss[lane] : 0.f;
    const float v2 = lane < k ? ss[k + lane] : 0.f;
    const int i1 = lane < k ? si[lane] : 0;
    const int i2 = lane < k ? si[k + lane] : 0;

    const float s0 = shfl_f32(v1, a0) + shfl_f32(v2, b0);
    const float s1 = shfl_f32(v1, a1) + shfl_f32(v2, b1);
    const int r0 = shfl_i32(i1, a0) * nk2 + shfl_i32(i2, b0);
    const int r1 = shfl_i32(i1, a1) * nk2 + shfl_i32(i2, b1);
    const bool ok0 = lane < P, ok1 = lane + 64 < P;
    const uint32_t h0 = ok0 ? float_key(s0) : 0u;
    const uint32_t h1 = ok1 ? float_key(s1) : 0u;
    const uint32_t l0 = ~uint32_t(r0), l1 = ~uint32_t(r1);

    // k-th largest score key, by bisection between a lower bound and the
    // largest key: the k candidates (a, 0), a < k, are all in the set, so the
    // k-th largest key is at least that of (k-1, 0), and the bits above the
    // highest one where the two bounds differ are fixed.
    const uint32_t hi = float_key(shfl_f32(v1, 0) + shfl_f32(v2, 0));
    const uint32_t lo = float_key(shfl_f32(v1, k - 1) + shfl_f32(v2, 0));
    const int top = hi == lo ? -1 : 31 - __builtin_clz(hi ^ lo);
    uint32_t thr = top < 0 ? lo : (lo & ~((2u << top) - 1u));
    for (int b = top; b >= 0; --b) {
      const uint32_t c = thr | (1u << b);
      if (popc64(ballot(h0 >= c)) + popc64(ballot(h1 >= c)) >= k) thr = c;
    }
    const int ngt = popc64(ballot(h0 > thr)) + popc64(ballot(h1 > thr));
    const int need = k - ngt;
    const bool e0 = h0 == thr, e1 = h1 == thr;
    uint32_t lthr = 0;
    if (popc64(ballot(e0)) + popc64(ballot(e1)) > need) {
      // equal scores at the cut: lowest rows (largest ~row) first
#pragma unroll
      for (int b = 31; b >= 0; --b) {
        const uint32_t c = lthr | (1u << b);
        if (popc64(ballot(e0 && l0 >= c)) + popc64(ballot(e1 && l1 >= c)) >= need) lthr = c;
      }
    }
    const bool sel0 = h0 > thr || (e0 && l0 >= lthr);
    const bool sel1 = h1 > thr || (e1 && l1 >= lthr);
    const uint64_t m0 = ballot(sel0), m1 = ballot(sel1);
    if (sel0) scr[lanes_below(m0)] = (uint64_t(h0) << 32) | l0;
    if (sel1) scr[popc64(m0) + lanes_below(m1)] = (uint64_t(h1) << 32) | l1;
    wave_lds_sync();
    uint64_t v = lane < k ? scr[lane] : 0ull;
    wave_lds_sync();
    v = sort32_desc_u64(v);

    const float sc = key_float(uint32_t(v >> 32));
    const int row = int(~uint32_t(v));
    const float smax = shfl_f32(sc, 0);
    const float e = lane < k ? expf((sc - smax) * inv_tau) : 0.f;
    const float sum = wave_sum_dpp(e);
    if (lane < k) {
      const int64_t o = it * k + lane;
      idx[o] = group_items ? int32_t(row + ((it / group_items) % group_count) * group_rows) : row;
      w[o] = e / sum;
      if (score) score[o] = sc;
    }
  }
}

}  // namespace

hipError_t launch_merge_softmax(hipStream_t s, const int32_t* sub_idx, const float* sub_score,
                                int64_t nitems, int k, int nk2, float inv_tau, int32_t* idx, float* w,
                                float* score, int64_t group_items, int64_t group_rows, int64_t group_count) {
  if (group_items > 0 && group_count < 1) return hipErrorInvalidValue;
  int64_t blocks = (nitems + kWavesPerBlock - 1) / kWavesPerBlock;
  if (blocks > 65536) blocks = 65536;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(merge_softmax_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, sub_idx, sub_score,
                     nitems, k, nk2, inv_tau, idx, w, score, group_items, group_rows, group_count);
  return hipGetLastError();
}

}  // namespace pkm
