// Step a5 for one (token, head) on one wave: k x k candidate merge, top-k of
// the candidates, softmax.
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
// can keep another of the equal-scoring rows than an exhaustive fp32 merge.)
// Each lane builds up to two candidates, the k-th largest 64-bit key (score
// key, ~row) is found by bisection with ballots, the k winners are compacted
// and sorted with a 32-lane bitonic network, and the softmax runs on the
// sorted lanes.  Used by the merge kernel and by the fused merge + gather.
#pragma once
#include "common.h"
#include "lane_ops.h"

namespace pkm {

__device__ __forceinline__ int merge_lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

__device__ __forceinline__ void merge_wave_lds_sync() {
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

// The candidate pairs (a | b << 8) of a workgroup, built by its first 64
// threads (lane a lists (a, b < k / (a + 1)) after those of every a' < a);
// the caller synchronises the workgroup before reading them.
__device__ __forceinline__ void merge_build_pairs(int k, uint16_t* pairs /*[128]*/, int* npairs) {
  if (threadIdx.x < 64) {
    const int a = threadIdx.x;
    const int cnt = a < k ? k / (a + 1) : 0;
    int x = cnt;
#pragma unroll
    for (int d = 1; d < 64; d <<= 1) {
      const int y = __shfl_up(x, d, 64);
      if (a >= d) x += y;
    }
    for (int b = 0; b < cnt; ++b) pairs[x - cnt + b] = uint16_t(a | (b << 8));
    if (a == 63) *npairs = x;
  }
}

// The lane's two candidate pairs (a0, b0), (a1, b1) out of P.
struct MergeLanePairs {
  int a0, b0, a1, b1, P;
};

__device__ __forceinline__ MergeLanePairs merge_lane_pairs(const uint16_t* pairs, int P) {
  const int lane = lane_id();
  const uint16_t pr0 = lane < P ? pairs[lane] : 0;
  const uint16_t pr1 = lane + 64 < P ? pairs[lane + 64] : 0;
  return MergeLanePairs{pr0 & 0xFF, pr0 >> 8, pr1 & 0xFF, pr1 >> 8, P};
}

// Item `it` (a (token, head)): lane s < k gets the s-th best row, its weight
// and its score.  scr: 64 words of LDS owned by the wave.
__device__ __forceinline__ void merge_item(const int32_t* __restrict__ sub_idx, const float* __restrict__ sub_score,
                                           int64_t it, int k, int nk2, float inv_tau, const MergeLanePairs& lp,
                                           uint64_t* scr, int& row_out, float& w_out, float& score_out) {
  const int lane = lane_id();
  const int32_t* si = sub_idx + it * 2 * k;
  const float* ss = sub_score + it * 2 * k;
  const float v1 = lane < k ? ss[lane] : 0.f;
  const float v2 = lane < k ? ss[k + lane] : 0.f;
  const int i1 = lane < k ? si[lane] : 0;
  const int i2 = lane < k ? si[k + lane] : 0;

  const float s0 = shfl_f32(v1, lp.a0) + shfl_f32(v2, lp.b0);
  const float s1 = shfl_f32(v1, lp.a1) + shfl_f32(v2, lp.b1);
  const int r0 = shfl_i32(i1, lp.a0) * nk2 + shfl_i32(i2, lp.b0);
  const int r1 = shfl_i32(i1, lp.a1) * nk2 + shfl_i32(i2, lp.b1);
  const bool ok0 = lane < lp.P, ok1 = lane + 64 < lp.P;
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
  if (sel0) scr[merge_lanes_below(m0)] = (uint64_t(h0) << 32) | l0;
  if (sel1) scr[popc64(m0) + merge_lanes_below(m1)] = (uint64_t(h1) << 32) | l1;
  merge_wave_lds_sync();
  uint64_t v = lane < k ? scr[lane] : 0ull;
  merge_wave_lds_sync();
  v = sort32_desc_u64(v);

  const float sc = key_float(uint32_t(v >> 32));
  const float smax = shfl_f32(sc, 0);
  const float e = lane < k ? expf((sc - smax) * inv_tau) : 0.f;
  const float sum = wave_sum_dpp(e);
  row_out = int(~uint32_t(v));
  w_out = e / sum;
  score_out = sc;
}

}  // namespace pkm
