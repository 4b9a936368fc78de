// Step a5: k x k candidate merge, top-k of the candidates, softmax, one wave
// per (token, head); the arithmetic is merge_item (merge_common.h).
#include "kernels.h"
#include "merge_common.h"

namespace pkm {

namespace {

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
  merge_build_pairs(k, pairs, &npairs);
  __syncthreads();
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  const MergeLanePairs lp = merge_lane_pairs(pairs, npairs);
  for (int64_t it = int64_t(blockIdx.x) * kWavesPerBlock + wave; it < nitems;
       it += int64_t(gridDim.x) * kWavesPerBlock) {
    int row;
    float wv, sc;
    merge_item(sub_idx, sub_score, it, k, nk2, inv_tau, lp, scratch[wave], row, wv, sc);
    if (lane < k) {
      const int64_t o = it * k + lane;
      idx[o] = group_items ? int32_t(row + ((it / group_items) % group_count) * group_rows) : row;
      w[o] = wv;
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
  // at most 8 blocks per CU: large launches loop (the pair table is built once per block)
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  }
  if (blocks > int64_t(cus) * 8) blocks = int64_t(cus) * 8;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(merge_softmax_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, sub_idx, sub_score,
                     nitems, k, nk2, inv_tau, idx, w, score, group_items, group_rows, group_count);
  return hipGetLastError();
}

}  // namespace pkm
