// Sparse backward (steps a7, a8, a9): gradient flows only through the
// selected rows and sub-keys ("Meta AI 可扩展内存层", section 6.1: only the
// activated key/value pairs accumulate gradient; section 9.2: back-propagate
// only at the selected positions; product-key paper summary, method details:
// only a few memory slots are updated).
//
//   dw[t,h,s] = <dY[t], V[r]>                       r = idx[t,h,s]
//   dV[r]    (+)= sum_{(t,h,s): idx = r} w[t,h,s] dY[t]
//   ds       = w (dw - sum_s w dw) / tau
//   dq1[t,h] = sum_s ds C[h, r/|C'|],  dq2[t,h] = sum_s ds C'[h, r%|C'|]
//   dC[h,i]  = sum_{(t,s): r/|C'| = i} ds q1[t,h],  likewise dC'
//
// value_grad walks the lookups grouped by row (a stable sort of the row ids),
// one wave per touched row: V[r] is read once and kept in registers, every
// lookup of r reads its dY row, produces dw with one wave reduction and adds
// w*dY into the row's fp32 gradient, which is written (or added) once.  The
// sub-key gradients use the same grouping keyed by sub-key.  A skewed workload
// makes some runs very long (thousands of lookups of one row, 10^5 of one
// sub-key); a plan kernel cuts those into fixed chunks, which the main launch
// processes first and in parallel with the short runs, each chunk's partial
// sum landing in its own slot; a short combine pass then adds each long run's
// slots in chunk order.  Every sum thus has a fixed order, so results are
// bit-identical from run to run.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int kVgU = 2;


// <a, v> over one 16-byte vector, accumulated into c.  bf16: v_dot2_f32_bf16 on
// packed pairs (products exact in fp32); fp32: four FMAs.
template <typename T>
__device__ __forceinline__ float dot16(const u32x4& a, const u32x4& v, float c);
template <>
__device__ __forceinline__ float dot16<bf16_t>(const u32x4& a, const u32x4& v, float c) {
  // whole-vector bit casts and shuffles: casting single elements of a u32x4 to
  // bf16x2 miscompiles here (every pair read the same register)
  const bf16x8 A = __builtin_bit_cast(bf16x8, a), B = __builtin_bit_cast(bf16x8, v);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 0, 1), __builtin_shufflevector(B, B, 0, 1), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 2, 3), __builtin_shufflevector(B, B, 2, 3), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 4, 5), __builtin_shufflevector(B, B, 4, 5), c, false);
  c = __builtin_amdgcn_fdot2_f32_bf16(__builtin_shufflevector(A, A, 6, 7), __builtin_shufflevector(B, B, 6, 7), c, false);
  return c;
}
template <>
__device__ __forceinline__ float dot16<float>(const u32x4& a, const u32x4& v, float c) {
  c = fmaf(__uint_as_float(a.x), __uint_as_float(v.x), c);
  c = fmaf(__uint_as_float(a.y), __uint_as_float(v.y), c);
  c = fmaf(__uint_as_float(a.z), __uint_as_float(v.z), c);
  c = fmaf(__uint_as_float(a.w), __uint_as_float(v.w), c);
  return c;
}

// Lookups of one row longer than this many entries are cut into chunks that
// separate waves process; their partial sums meet in a fixed order.
constexpr int kVgChunk = 256;

struct VgArgs {
  const int32_t* seg_start;
  const int64_t* nseg;
  const uint32_t* sorted_rows;
  const int32_t* sorted_c;
  const float* w;
  const void* dY;
  const void* V;
  float* dV;
  float* dw;
  uint32_t R;  // lookups per token (h*k)
  int nvec;    // 16-byte vectors per row
  int accumulate;
  // long rows
  const int2* chunk_list;   // (row run u, chunk j): list entry i owns partial slot i
  const int2* long_list;    // (row run u, first slot) of every run longer than kVgChunk
  const uint32_t* counts;   // [0] chunks listed, [1] long runs listed
  float* partial;           // [2 N / kVgChunk + 2, d_v] partial sums
};

// The wave's lanes own 16-byte vectors l, l+64, ... of a row; the first NVL-1
// are in range for every lane (the launcher picks NVL so), only the last one is
// predicated: out-of-range lanes read vector 0 instead (discarded), so every
// load is issued unconditionally.
template <int NVL>
struct LaneVecs {
  int voff[NVL];
  bool last_ok;
  __device__ __forceinline__ LaneVecs(int nvec, int lane) {
    last_ok = (NVL - 1) * 64 + lane < nvec;
#pragma unroll
    for (int m = 0; m < NVL; ++m) voff[m] = (m < NVL - 1 || last_ok) ? (m * 64 + lane) * 16 : 0;
  }
};

// g += sum over sorted lookups [lo, hi) of w * dY[t]; dw of each lookup = <dY[t], V[r]>.
// Each lookup costs one dY row read, NVL dot products, one DPP wave reduction and
// the fp32 FMAs of w*dY; two lookups are in flight per step.
template <typename T, int NVL>
__device__ __forceinline__ void vg_accumulate(const VgArgs& a, const LaneVecs<NVL>& lv, const u32x4* vr, int lo,
                                              int hi, float (*g)[Vec16<T>::N]) {
  constexpr int E = Vec16<T>::N;
  const int lane = lane_id();
  const size_t row_bytes = size_t(a.nvec) * 16;
  const char* Yb = reinterpret_cast<const char*>(a.dY);
  for (int c0 = lo; c0 < hi; c0 += 64) {
    const int n = min(64, hi - c0);
    const int my_c = lane < n ? a.sorted_c[c0 + lane] : 0;
    const float my_w = lane < n ? a.w[my_c] : 0.f;
    float my_dw = 0.f;
    for (int j = 0; j < n; j += kVgU) {
      u32x4 buf[kVgU][NVL];
#pragma unroll
      for (int uu = 0; uu < kVgU; ++uu) {
        const int jj = j + uu < n ? j + uu : n - 1;
        const uint32_t c = uint32_t(__builtin_amdgcn_readlane(my_c, jj));
        const char* yrow = Yb + size_t(c / a.R) * row_bytes;
#pragma unroll
        for (int m = 0; m < NVL; ++m) buf[uu][m] = ld16(yrow + lv.voff[m]);
      }
#pragma unroll
      for (int uu = 0; uu < kVgU; ++uu) {
        if (j + uu < n) {  // wave-uniform
          const float wt = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(my_w), j + uu));
          float part = 0.f;
#pragma unroll
          for (int m = 0; m < NVL; ++m) {
            part = dot16<T>(buf[uu][m], vr[m], part);
            float f[E];
            Vec16<T>::widen(buf[uu][m], f);
#pragma unroll
            for (int e = 0; e < E; ++e) g[m][e] = fmaf(wt, f[e], g[m][e]);
          }
          const float sm = wave_sum_dpp(part);
          if (lane == j + uu) my_dw = sm;
        }
      }
    }
    if (lane < n) a.dw[my_c] = my_dw;
  }
}

template <typename T, int NVL>
__device__ __forceinline__ void vg_load_row(const VgArgs& a, const LaneVecs<NVL>& lv, uint32_t r, u32x4* vr) {
  const char* vrow = reinterpret_cast<const char*>(a.V) + size_t(r) * size_t(a.nvec) * 16;
#pragma unroll
  for (int m = 0; m < NVL; ++m) vr[m] = ld16_nt(vrow + lv.voff[m]);
  if (!lv.last_ok) vr[NVL - 1] = u32x4{0, 0, 0, 0};
}

// dst[lane's part] = g (+ old dst when add_old)
template <typename T, int NVL>
__device__ __forceinline__ void vg_store(const LaneVecs<NVL>& lv, float* drow, const float (*g)[Vec16<T>::N],
                                         bool add_old) {
  constexpr int E = Vec16<T>::N;
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    if (m == NVL - 1 && !lv.last_ok) continue;
    float* p = drow + (lv.voff[m] / 16) * E;
#pragma unroll
    for (int q4 = 0; q4 < E / 4; ++q4) {
      f32x4 o = {g[m][q4 * 4 + 0], g[m][q4 * 4 + 1], g[m][q4 * 4 + 2], g[m][q4 * 4 + 3]};
      if (add_old) o += *reinterpret_cast<const f32x4*>(p + q4 * 4);
      *reinterpret_cast<f32x4*>(p + q4 * 4) = o;
    }
  }
}

template <typename T, int NVL>
__device__ __forceinline__ void vg_add_from(const LaneVecs<NVL>& lv, const float* src, float (*g)[Vec16<T>::N]) {
  constexpr int E = Vec16<T>::N;
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const float* p = src + (lv.voff[m] / 16) * E;
#pragma unroll
    for (int q4 = 0; q4 < E / 4; ++q4) {
      const f32x4 o = *reinterpret_cast<const f32x4*>(p + q4 * 4);
      g[m][q4 * 4 + 0] += o.x;
      g[m][q4 * 4 + 1] += o.y;
      g[m][q4 * 4 + 2] += o.z;
      g[m][q4 * 4 + 3] += o.w;
    }
  }
}

// MODE 0: one wave per work item, a resident grid striding over the items:
//         first the chunks of the long runs (partial sums into their slots),
//         then the runs of at most kVgChunk lookups, whose value row is read
//         once and gradient row written (or added) once.
// MODE 1: one wave per long run: its slots added in chunk order into dV.
template <typename T, int NVL, int MODE>
__global__ __launch_bounds__(256) void value_grad_kernel(VgArgs a) {
  constexpr int E = Vec16<T>::N;
  const int lane = lane_id();
  const int64_t gw = (int64_t(blockIdx.x) * blockDim.x + threadIdx.x) >> 6;
  const int64_t nw = (int64_t(gridDim.x) * blockDim.x) >> 6;
  const int dv = a.nvec * E;
  const LaneVecs<NVL> lv(a.nvec, lane);
  if (MODE == 1) {
    const int64_t nlong = a.counts[1];
    for (int64_t it = gw; it < nlong; it += nw) {
      const int2 e = a.long_list[it];
      const int lo = a.seg_start[e.x], hi = a.seg_start[e.x + 1];
      const uint32_t r = a.sorted_rows[lo];
      float g[NVL][E];
#pragma unroll
      for (int m = 0; m < NVL; ++m)
#pragma unroll
        for (int q = 0; q < E; ++q) g[m][q] = 0.f;
      const int nch = (hi - lo + kVgChunk - 1) / kVgChunk;
      for (int j = 0; j < nch; ++j) vg_add_from<T, NVL>(lv, a.partial + size_t(e.y + j) * dv, g);
      vg_store<T, NVL>(lv, a.dV + size_t(r) * dv, g, a.accumulate != 0);
    }
    return;
  }
  const int64_t nchunks = a.counts[0];
  const int64_t nitems = nchunks + *a.nseg;
  for (int64_t it = gw; it < nitems; it += nw) {
    const bool chunk = it < nchunks;  // wave-uniform
    int u, j = 0;
    if (chunk) {
      const int2 e = a.chunk_list[it];
      u = e.x;
      j = e.y;
    } else {
      u = int(it - nchunks);
    }
    const int lo = a.seg_start[u], hi = a.seg_start[u + 1];
    if (!chunk && hi - lo > kVgChunk) continue;  // wave-uniform: listed as chunks
    const uint32_t r = a.sorted_rows[lo];
    u32x4 vr[NVL];
    vg_load_row<T, NVL>(a, lv, r, vr);
    float g[NVL][E];
#pragma unroll
    for (int m = 0; m < NVL; ++m)
#pragma unroll
      for (int q = 0; q < E; ++q) g[m][q] = 0.f;
    const int clo = lo + j * kVgChunk;
    const int chi = chunk ? min(hi, clo + kVgChunk) : hi;
    vg_accumulate<T, NVL>(a, lv, vr, clo, chi, g);
    if (chunk)
      vg_store<T, NVL>(lv, a.partial + size_t(it) * dv, g, false);
    else
      vg_store<T, NVL>(lv, a.dV + size_t(r) * dv, g, a.accumulate != 0);
  }
}

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
      uint64_t mm = m1;
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        const int is = __builtin_amdgcn_readlane(i, b);
        load4_acc(Ch + size_t(is) * half + ch * 4, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s1), b)), a1);
      }
      mm = m2;
      while (mm) {
        const int b = __builtin_ctzll(mm);
        mm &= mm - 1;
        const int js = __builtin_amdgcn_readlane(j, b);
        load4_acc(Cph + size_t(js) * half + ch * 4, __int_as_float(__builtin_amdgcn_readlane(__float_as_int(s2), b)), a2);
      }
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

size_t value_grad_aux_bytes(int64_t nitems, int d_value) {
  const int64_t slots = 2 * (nitems / kVgChunk) + 2;  // chunks of runs longer than a chunk: < 2 N / kVgChunk
  return size_t(slots) * (size_t(d_value) * 4 + 8 + 8) + 64;
}

hipError_t launch_value_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg,
                             int64_t nitems, const uint32_t* sorted_rows, const int32_t* sorted_c, const float* w,
                             const void* dY, const void* V, float* dV, float* dw, int R, int d_value,
                             bool accumulate, void* aux) {
  const int elem = dtype == kBF16 ? 2 : 4;
  const int nvec = d_value * elem / 16;
  const int per_lane = (nvec + 63) / 64;
  const int64_t slots = 2 * (nitems / kVgChunk) + 2;
  char* ap = static_cast<char*>(aux);
  VgArgs a;
  a.seg_start = seg_start;
  a.nseg = nseg;
  a.sorted_rows = sorted_rows;
  a.sorted_c = sorted_c;
  a.w = w;
  a.dY = dY;
  a.V = V;
  a.dV = dV;
  a.dw = dw;
  a.R = uint32_t(R);
  a.nvec = nvec;
  a.accumulate = int(accumulate);
  uint32_t* counts = reinterpret_cast<uint32_t*>(ap);
  a.counts = counts;
  a.partial = reinterpret_cast<float*>(ap + 64);
  int2* chunk_list = reinterpret_cast<int2*>(ap + 64 + size_t(slots) * d_value * 4);
  int2* long_list = chunk_list + slots;
  a.chunk_list = chunk_list;
  a.long_list = long_list;
  hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, counts, 2);
  int64_t pb = (nitems + 255) / 256;
  if (pb > 4096) pb = 4096;
  if (pb < 1) pb = 1;
  hipLaunchKernelGGL(long_run_plan_kernel, dim3(unsigned(pb)), dim3(256), 0, s, seg_start, nseg, kVgChunk,
                     static_cast<const uint32_t*>(nullptr), 0u, chunk_list, long_list, counts);
  const dim3 block(256);
  const dim3 grid_long(grid_waves(slots, 1024));
#define PKM_VG(TT, NV)                                                                                    \
  do {                                                                                                    \
    const dim3 grid(resident_grid(reinterpret_cast<const void*>(value_grad_kernel<TT, NV, 0>), nitems));  \
    hipLaunchKernelGGL((value_grad_kernel<TT, NV, 0>), grid, block, 0, s, a);                             \
    hipLaunchKernelGGL((value_grad_kernel<TT, NV, 1>), grid_long, block, 0, s, a);                        \
  } while (0)
  if (dtype == kBF16) {
    if (per_lane <= 1) PKM_VG(bf16_t, 1);
    else if (per_lane == 2) PKM_VG(bf16_t, 2);
    else if (per_lane == 3) PKM_VG(bf16_t, 3);
    else if (per_lane == 4) PKM_VG(bf16_t, 4);
    else return hipErrorInvalidValue;
  } else {
    if (per_lane <= 1) PKM_VG(float, 1);
    else if (per_lane == 2) PKM_VG(float, 2);
    else if (per_lane == 3) PKM_VG(float, 3);
    else if (per_lane == 4) PKM_VG(float, 4);
    else return hipErrorInvalidValue;
  }
#undef PKM_VG
  return hipGetLastError();
}

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
