// Pieces shared by the sparse-gradient kernels (value and sub-key gradients):
// the long-run plan kernel, a small counter-clearing kernel and the grid
// sizing helpers.  Internal to the library; each translation unit gets its own
// copy (anonymous namespace).
#pragma once
#include "common.h"
#include "kernels.h"

namespace pkm {
namespace {

// Lists the runs longer than `chunk` entries, every chunk of them (run u,
// chunk j) in chunk_list and (u, first list entry) in long_list.  List order
// is free: a chunk's partial sum goes to the slot of its list entry and a long
// run adds its slots in chunk order, so results do not depend on it.  Runs
// whose key is >= nvalid are skipped (keys == nullptr: none is).
__global__ __launch_bounds__(256) void long_run_plan_kernel(const int32_t* __restrict__ seg_start,
                                                            const int64_t* __restrict__ nseg_p, int chunk,
                                                            const uint32_t* __restrict__ keys, uint32_t nvalid,
                                                            int2* __restrict__ chunk_list,
                                                            int2* __restrict__ long_list,
                                                            uint32_t* __restrict__ counts) {
  const int64_t nseg = *nseg_p;
  for (int64_t u = int64_t(blockIdx.x) * 256 + threadIdx.x; u < nseg; u += int64_t(gridDim.x) * 256) {
    const int lo = seg_start[u];
    const int len = seg_start[u + 1] - lo;
    if (len > chunk && (keys == nullptr || keys[lo] < nvalid)) {
      const int nch = (len + chunk - 1) / chunk;
      const uint32_t base = atomicAdd(&counts[0], uint32_t(nch));
      for (int j = 0; j < nch; ++j) chunk_list[base + j] = make_int2(int(u), j);
      long_list[atomicAdd(&counts[1], 1u)] = make_int2(int(u), int(base));
    }
  }
}

__global__ void zero_u32_kernel(uint32_t* p, int n) {
  if (threadIdx.x < n) p[threadIdx.x] = 0u;
}

// As many 256-thread blocks as the device holds at once, but no more than one
// wave per item.
unsigned resident_grid(const void* fn, int64_t items) {
  int dev = 0, cus = 0, per_cu = 0;
  if (hipGetDevice(&dev) != hipSuccess ||
      hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
      hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, fn, 256, 0) != hipSuccess || per_cu < 1 || cus < 1) {
    cus = 256;
    per_cu = 2;
  }
  int64_t b = int64_t(cus) * per_cu;
  const int64_t need = (items + 3) / 4;
  if (b > need) b = need;
  if (b < 1) b = 1;
  return unsigned(b);
}

inline unsigned grid_waves(int64_t items, int64_t cap_blocks = 4096) {
  int64_t b = (items + 3) / 4;
  if (b > cap_blocks) b = cap_blocks;
  if (b < 1) b = 1;
  return unsigned(b);
}

}  // namespace
}  // namespace pkm
