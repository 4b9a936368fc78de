// Softmax backward and the query / sub-key gradients (steps a7 and a9): the
// gradient reaches only the selected sub-keys ("Meta AI 可扩展内存层", section
// 9.2: back-propagate only at the selected positions; section 6.1: only the
// activated keys accumulate gradient).
//
//   ds       = w (dw - sum_s w dw) / tau
//   dq1[t,h] = sum_s ds C[h, r/|C'|],  dq2[t,h] = sum_s ds C'[h, r%|C'|]
//   dC[h,i]  = sum_{(t,s): r/|C'| = i} ds q1[t,h],  likewise dC'
//
// The sub-key gradients use the same grouping as the value gradient, keyed by
// sub-key (a stable sort), one block per sub-key; sub-keys with very many
// entries are cut into chunks combined in chunk order, so sums run in a fixed
// order and results are bit-identical from run to run.
#include "sparse_common.h"

namespace pkm {

namespace {

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

// a += sum over the set bits b of mask (slots, in order) of coef[b] * rows[id[b]][4 ch .. 4 ch + 3],
// eight rows in flight at a time (padding entries repeat the batch's first row
// with coefficient 0).  mask, id and coef are wave-uniform per slot.
template <typename T>
__device__ __forceinline__ void gather_rows(uint64_t mask, int id, float coef, const T* rows, int half, int ch,
                                            float* a) {
  constexpr int U = 8;
  while (mask) {
    int r[U];
    float cf[U];
    const int b0 = __builtin_ctzll(mask);
#pragma unroll
    for (int u = 0; u < U; ++u) {
      const int b = mask ? __builtin_ctzll(mask) : b0;
      cf[u] = mask ? __int_as_float(__builtin_amdgcn_readlane(__float_as_int(coef), b)) : 0.f;
      r[u] = __builtin_amdgcn_readlane(id, b);
      mask &= mask - 1;
    }
    float f[U][4];
#pragma unroll
    for (int u = 0; u < U; ++u) load4(rows + size_t(r[u]) * half + ch * 4, f[u]);
#pragma unroll
    for (int u = 0; u < U; ++u)
#pragma unroll
      for (int e = 0; e < 4; ++e) a[e] = fmaf(cf[u], f[u][e], a[e]);
  }
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
      gather_rows<T>(m1, i, s1, Ch, half, ch, a1);
      gather_rows<T>(m2, j, s2, Cph, half, ch, a2);
      if (chb + lane < nch) {
        *reinterpret_cast<f32x4*>(o + ch * 4) = f32x4{a1[0], a1[1], a1[2], a1[3]};
        *reinterpret_cast<f32x4*>(o + half + ch * 4) = f32x4{a2[0], a2[1], a2[2], a2[3]};
      }
    }
  }
}

constexpr int kSkU = 8;
constexpr int kSkWaves = 4;
// Sub-keys with more entries than this are cut into chunks processed by
// separate blocks; their partial sums meet in a fixed order.
constexpr int kSkChunk = 2048;

struct SkArgs {
  const int32_t* seg_start;
  const int64_t* nseg;
  const uint32_t* sorted_keys;
  const int32_t* sorted_c;
  const float* coef;
  const void* q;
  float* dC;
  int heads, dq, k, half_sel, nkeys;
  const int2* chunk_list;    // (run u, chunk j): list entry i owns partial slot i
  const int2* long_list;     // (run u, first slot) of every run longer than kSkChunk
  const uint32_t* counts;    // [0] chunks listed, [1] long runs listed
  float* partial;            // [2 N / kSkChunk + 2, dq/2] partial sums
};

// One 4-wave block per work item (grid-stride): dC[key] = sum over the key's
// entries of coef * q_half[t, h].  Wave v takes entries v, v+4, ... in batches
// of 8 rows, and the four partial sums are added in wave order through LDS.
// MODE 0: first the chunks of the long runs (into their partial slots), then
//         the runs of at most kSkChunk entries (into dC).
// MODE 1: one block per long run: its slots added in chunk order into dC.
template <typename T, int MODE>
__global__ __launch_bounds__(256) void subkey_grad_kernel(SkArgs a) {
  __shared__ f32x4 part[kSkWaves][64];
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  const int half = a.dq / 2;
  const int nch = half / 4;
  const int F = a.heads * a.dq;
  const uint32_t nvalid = uint32_t(a.heads) * uint32_t(a.nkeys);
  const int kh = a.k * a.heads;
  if (MODE == 1) {
    const int64_t nlong = a.counts[1];
    for (int64_t it = blockIdx.x; it < nlong; it += gridDim.x) {
      const int2 e = a.long_list[it];
      const int lo = a.seg_start[e.x], hi = a.seg_start[e.x + 1];
      const uint32_t key = a.sorted_keys[lo];
      const int nchk = (hi - lo + kSkChunk - 1) / kSkChunk;
      for (int ch = threadIdx.x; ch < nch; ch += blockDim.x) {
        f32x4 tot = {0.f, 0.f, 0.f, 0.f};
        for (int j = 0; j < nchk; ++j) tot += *reinterpret_cast<const f32x4*>(a.partial + size_t(e.y + j) * half + ch * 4);
        *reinterpret_cast<f32x4*>(a.dC + size_t(key) * half + ch * 4) = tot;
      }
    }
    return;
  }
  const int64_t nchunks = a.counts[0];
  const int64_t nitems = nchunks + *a.nseg;
  for (int64_t it = blockIdx.x; it < nitems; it += gridDim.x) {
    const bool chunk = it < nchunks;  // block-uniform
    int u, j = 0;
    if (chunk) {
      const int2 e = a.chunk_list[it];
      u = e.x;
      j = e.y;
    } else {
      u = int(it - nchunks);
    }
    const int lo = a.seg_start[u], hi = a.seg_start[u + 1];
    const uint32_t key = a.sorted_keys[lo];
    if (key >= nvalid) continue;                      // block-uniform: the sentinel run (repeated sub-keys)
    if (!chunk && hi - lo > kSkChunk) continue;       // block-uniform: listed as chunks
    const int clo = lo + j * kSkChunk;
    const int chi = chunk ? min(hi, clo + kSkChunk) : hi;
    const int hh = int(key / uint32_t(a.nkeys));
    const T* qh = static_cast<const T*>(a.q) + size_t(hh) * a.dq + size_t(a.half_sel) * half;
    for (int chb = 0; chb < nch; chb += 64) {
      const int ch = min(chb + lane, nch - 1);
      float acc[4] = {0.f, 0.f, 0.f, 0.f};
      for (int c0 = clo + wave; c0 < chi; c0 += kSkWaves * 64) {
        // entries c0, c0+4, ..., one per lane
        const int e = c0 + lane * kSkWaves;
        const int my_c = e < chi ? a.sorted_c[e] : 0;
        const float my_d = e < chi ? a.coef[my_c] : 0.f;
        const int n = min(64, (chi - c0 + kSkWaves - 1) / kSkWaves);
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
              for (int q4 = 0; q4 < 4; ++q4) acc[q4] = fmaf(d, f[uu][q4], acc[q4]);
            }
          }
        }
      }
      part[wave][lane] = f32x4{acc[0], acc[1], acc[2], acc[3]};
      __syncthreads();
      if (wave == 0 && chb + lane < nch) {
        f32x4 tot = part[0][lane];
#pragma unroll
        for (int v = 1; v < kSkWaves; ++v) tot += part[v][lane];
        float* dst = chunk ? a.partial + size_t(it) * half : a.dC + size_t(key) * half;
        *reinterpret_cast<f32x4*>(dst + ch * 4) = tot;
      }
      __syncthreads();
    }
  }
}

}  // namespace

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

size_t subkey_grad_aux_bytes(int64_t nitems, int dq) {
  const int64_t slots = 2 * (nitems / kSkChunk) + 2;  // chunks of runs longer than a chunk: < 2 N / kSkChunk
  return size_t(slots) * (size_t(dq / 2) * 4 + 8 + 8) + 64;
}

hipError_t launch_subkey_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg, int64_t nsub,
                              int64_t nitems, const uint32_t* sorted_keys, const int32_t* sorted_c, const float* coef,
                              const void* q, int heads, int dq, int k, int half_sel, int nkeys, float* dC, void* aux) {
  const int64_t slots = 2 * (nitems / kSkChunk) + 2;
  const int half = dq / 2;
  char* ap = static_cast<char*>(aux);
  SkArgs a;
  a.seg_start = seg_start;
  a.nseg = nseg;
  a.sorted_keys = sorted_keys;
  a.sorted_c = sorted_c;
  a.coef = coef;
  a.q = q;
  a.dC = dC;
  a.heads = heads;
  a.dq = dq;
  a.k = k;
  a.half_sel = half_sel;
  a.nkeys = nkeys;
  uint32_t* counts = reinterpret_cast<uint32_t*>(ap);
  a.counts = counts;
  a.partial = reinterpret_cast<float*>(ap + 64);
  int2* chunk_list = reinterpret_cast<int2*>(ap + 64 + size_t(slots) * half * 4);
  int2* long_list = chunk_list + slots;
  a.chunk_list = chunk_list;
  a.long_list = long_list;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, counts, 2);
  int64_t pb = (nsub + 1 + 255) / 256;  // at most one run per distinct sub-key (+ the sentinel run)
  if (pb > 4096) pb = 4096;
  hipLaunchKernelGGL(long_run_plan_kernel, dim3(unsigned(pb)), dim3(256), 0, s, seg_start, nseg, kSkChunk,
                     sorted_keys, uint32_t(heads) * uint32_t(nkeys), chunk_list, long_list, counts);
  // one block per run (at most one per sub-key, plus the sentinel) or chunk (< 2 N / kSkChunk)
  int64_t blocks = nsub + 1 + slots;
  if (blocks > 8192) blocks = 8192;
  int64_t lblocks = slots < 4096 ? slots : 4096;
  const dim3 grid{unsigned(blocks), 1, 1}, lgrid{unsigned(lblocks), 1, 1}, block{256, 1, 1};
  if (dtype == kBF16) {
    hipLaunchKernelGGL((subkey_grad_kernel<bf16_t, 0>), grid, block, 0, s, a);
    hipLaunchKernelGGL((subkey_grad_kernel<bf16_t, 1>), lgrid, block, 0, s, a);
  } else {
    hipLaunchKernelGGL((subkey_grad_kernel<float, 0>), grid, block, 0, s, a);
    hipLaunchKernelGGL((subkey_grad_kernel<float, 1>), lgrid, block, 0, s, a);
  }
  return hipGetLastError();
}

}  // namespace pkm
