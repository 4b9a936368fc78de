// Value gradient (steps a7 dw and a8): gradient flows only into the selected
// value rows ("Meta AI 可扩展内存层", section 6.1: only the activated key/value
// pairs accumulate gradient; section 9.2: back-propagate only at the selected
// positions; product-key paper summary, method details: only a few memory
// slots are updated).
//
//   dw[t,h,s] = <dY[t], V[r]>                       r = idx[t,h,s]
//   dV[r]    (+)= sum_{(t,h,s): idx = r} w[t,h,s] dY[t]
//
// value_grad walks the lookups grouped by row (a stable sort of the row ids),
// one wave per touched row: V[r] is read once and kept in registers, every
// lookup of r reads its dY row, produces dw with one wave reduction and adds
// w*dY into the row's fp32 gradient, which is written (or added) once.  A
// skewed workload makes some rows very long (thousands of lookups); a plan
// kernel cuts those into fixed chunks, which the main launch processes first
// and in parallel with the short runs, each chunk's partial sum landing in its
// own slot; a short combine pass then adds each long run's slots in chunk
// order.  Every sum thus has a fixed order, so results are bit-identical from
// run to run.
//
// Optional fused optimizer step ("Meta AI 可扩展内存层", section 6.3: Adam
// moments kept only for the parameters that got gradient, a learning rate of
// its own for the value table): instead of writing dV, each touched row's
// gradient g of this call updates its moments m, v and the row itself,
//   m = b1 m + (1-b1) g,  v = b2 v + (1-b2) g^2,
//   V = V - lr/(1-b1^t) * m / (sqrt(v)/sqrt(1-b2^t) + eps)   (t: global step),
// in the same pass that read the row for dw (so dw always sees the old row);
// rows cut into chunks are updated by the combine launch, after every chunk
// has read the old row.
#include "sparse_common.h"

namespace pkm {

namespace {

constexpr int kVgU = 4;  // dY rows in flight per wave
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

// Lookups of one row longer than kVgChunk entries are cut into chunks that
// separate waves process; their partial sums meet in a fixed order.

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
  // fused Adam step (value_grad_kernel<..., ADAM = true>): V is written in place
  void* Vout;
  float* am;
  float* av;
  float b1, b2, eps;
  float step_size;     // lr / (1 - b1^t); the plain learning rate when sgd
  float inv_sqrt_bc2;  // 1 / sqrt(1 - b2^t)
  int sgd;             // plain gradient step V -= step_size * g (no moments)
  int32_t* slot;       // moments in pool slots (VgAdam::slot); null: dense moment tables
  int64_t capacity;
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
// the fp32 FMAs of w*dY; kVgU lookups are in flight per step.
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
          if (!a.sgd) {  // wave-uniform: the plain step has no use for dw
            const float sm = wave_sum_dpp(part);
            if (lane == j + uu) my_dw = sm;
          }
        }
      }
    }
    if (!a.sgd && lane < n) a.dw[my_c] = my_dw;
  }
}

template <typename T, int NVL>
__device__ __forceinline__ void vg_load_row(const VgArgs& a, const LaneVecs<NVL>& lv, uint32_t r, u32x4* vr) {
  const char* vrow = reinterpret_cast<const char*>(a.V) + size_t(r) * size_t(a.nvec) * 16;
#pragma unroll
  for (int m = 0; m < NVL; ++m) vr[m] = ld16_nt(vrow + lv.voff[m]);
  if (!lv.last_ok) vr[NVL - 1] = u32x4{0, 0, 0, 0};
}

// The fp32 rows (dV, the chunk partial sums, the Adam moments) are each read
// and written once per call: non-temporal accesses keep them from displacing
// the dY rows, which every lookup of a token reads again (measured: 4.50 ->
// 4.34 ms for the value gradient, 9.25 -> 7.77 ms with the Adam step, paper
// scale).
__device__ __forceinline__ f32x4 ld16f_nt(const float* p) {
  return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void st16f_nt(float* p, const f32x4& v) {
  __builtin_nontemporal_store(v, reinterpret_cast<f32x4*>(p));
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
      if (add_old) o += ld16f_nt(p + q4 * 4);
      st16f_nt(p + q4 * 4, o);
    }
  }
}

// dst = the lane's part of an fp32 row (zeros for the out-of-range last vector)
template <typename T, int NVL>
__device__ __forceinline__ void vg_load_f32(const LaneVecs<NVL>& lv, const float* src, float (*dst)[Vec16<T>::N]) {
  constexpr int E = Vec16<T>::N;
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    const bool ok = m < NVL - 1 || lv.last_ok;
    const float* p = src + (lv.voff[m] / 16) * E;
#pragma unroll
    for (int q4 = 0; q4 < E / 4; ++q4) {
      const f32x4 o = ok ? ld16f_nt(p + q4 * 4) : f32x4{0.f, 0.f, 0.f, 0.f};
      dst[m][q4 * 4 + 0] = o.x;
      dst[m][q4 * 4 + 1] = o.y;
      dst[m][q4 * 4 + 2] = o.z;
      dst[m][q4 * 4 + 3] = o.w;
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
      const f32x4 o = ld16f_nt(p + q4 * 4);
      g[m][q4 * 4 + 0] += o.x;
      g[m][q4 * 4 + 1] += o.y;
      g[m][q4 * 4 + 2] += o.z;
      g[m][q4 * 4 + 3] += o.w;
    }
  }
}

// Adam step of row r from its gradient g: moments read, updated and written
// back, the row (old value in vr, storage packing) moved and stored.
template <typename T, int NVL>
__device__ __forceinline__ void vg_adam_row(const VgArgs& a, const LaneVecs<NVL>& lv, uint32_t r, const u32x4* vr,
                                            const float (*g)[Vec16<T>::N]) {
  constexpr int E = Vec16<T>::N;
  const size_t dv = size_t(a.nvec) * E;
  char* Vrow = reinterpret_cast<char*>(a.Vout) + size_t(r) * size_t(a.nvec) * 16;
  if (a.sgd) {  // wave-uniform: V -= lr * g
#pragma unroll
    for (int m = 0; m < NVL; ++m) {
      if (m == NVL - 1 && !lv.last_ok) continue;
      float old[E], nv[E];
      Vec16<T>::widen(vr[m], old);
#pragma unroll
      for (int e = 0; e < E; ++e) nv[e] = old[e] - a.step_size * g[m][e];
      st16(Vrow + lv.voff[m], Vec16<T>::narrow(nv));
    }
    return;
  }
  size_t prow = r;
  bool fresh = false;
  if (a.slot) {  // wave-uniform: the row's entry of the slot map
    const int32_t e = a.slot[r];
    if (e == -1) return;  // refused a slot: not stepped
    const int64_t sl = e >= 0 ? int64_t(e) : -2 - int64_t(e);
    if (sl >= a.capacity) return;
    prow = size_t(sl);
    fresh = e < -1;
  }
  float* mrow = a.am + prow * dv;
  float* vrow = a.av + prow * dv;
  float m0[NVL][E], v0[NVL][E];
  if (fresh) {  // a row's first step: zero moments, the pool row is not read
#pragma unroll
    for (int m = 0; m < NVL; ++m)
#pragma unroll
      for (int e = 0; e < E; ++e) m0[m][e] = v0[m][e] = 0.f;
  } else {
    vg_load_f32<T, NVL>(lv, mrow, m0);
    vg_load_f32<T, NVL>(lv, vrow, v0);
  }
#pragma unroll
  for (int m = 0; m < NVL; ++m) {
    if (m == NVL - 1 && !lv.last_ok) continue;
    float old[E], nv[E];
    Vec16<T>::widen(vr[m], old);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const float gm = g[m][e];
      const float m1 = a.b1 * m0[m][e] + (1.0f - a.b1) * gm;
      const float v1 = a.b2 * v0[m][e] + (1.0f - a.b2) * (gm * gm);
      m0[m][e] = m1;
      v0[m][e] = v1;
      nv[e] = old[e] - a.step_size * m1 / (__builtin_sqrtf(v1) * a.inv_sqrt_bc2 + a.eps);
    }
    st16(Vrow + lv.voff[m], Vec16<T>::narrow(nv));
  }
  vg_store<T, NVL>(lv, mrow, m0, false);
  vg_store<T, NVL>(lv, vrow, v0, false);
  if (fresh && lane_id() == 0) a.slot[r] = int32_t(prow);
}

// MODE 0: one wave per work item, a resident grid striding over the items:
//         first the chunks of the long runs (partial sums into their slots),
//         then the runs of at most kVgChunk lookups, whose value row is read
//         once and gradient row written (or added) once.
// MODE 1: one wave per long run: its slots added in chunk order into dV.
// ADAM: the row's gradient drives the Adam step (vg_adam_row) instead of dV.
template <typename T, int NVL, int MODE, bool ADAM>
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
      if constexpr (ADAM) {
        u32x4 vr[NVL];
        vg_load_row<T, NVL>(a, lv, r, vr);
        vg_adam_row<T, NVL>(a, lv, r, vr, g);
      } else {
        vg_store<T, NVL>(lv, a.dV + size_t(r) * dv, g, a.accumulate != 0);
      }
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
    // the old gradient row of a short run is fetched now, beside the value
    // row, so that its latency overlaps the lookups; it is added to the sum at
    // the end (the same order of additions as reading it there)
    const bool add_old = !ADAM && !chunk && a.accumulate != 0;  // wave-uniform
    float old[NVL][E];
    if (add_old) vg_load_f32<T, NVL>(lv, a.dV + size_t(r) * dv, old);
    float g[NVL][E];
#pragma unroll
    for (int m = 0; m < NVL; ++m)
#pragma unroll
      for (int q = 0; q < E; ++q) g[m][q] = 0.f;
    const int clo = lo + j * kVgChunk;
    const int chi = chunk ? min(hi, clo + kVgChunk) : hi;
    vg_accumulate<T, NVL>(a, lv, vr, clo, chi, g);
    if (chunk) {
      vg_store<T, NVL>(lv, a.partial + size_t(it) * dv, g, false);
    } else if constexpr (ADAM) {
      vg_adam_row<T, NVL>(a, lv, r, vr, g);
    } else {
      if (add_old) {
#pragma unroll
        for (int m = 0; m < NVL; ++m)
#pragma unroll
          for (int q = 0; q < E; ++q) g[m][q] += old[m][q];
      }
      vg_store<T, NVL>(lv, a.dV + size_t(r) * dv, g, false);
    }
  }
}

// Slot hand-out of the moment pool (VgAdam::slot): the touched rows (sorted,
// distinct) are cut into kRsBlocks equal ranges; a first launch counts each
// range's rows without a slot, a second gives them slots in row order, each
// block starting after the new rows of the ranges before it.
constexpr int kRsBlocks = 512;
constexpr int kRsThreads = 256;
constexpr int kRsWaves = kRsThreads / 64;

__device__ __forceinline__ void rs_range(const int64_t* n_touched, int64_t* lo, int64_t* hi) {
  const int64_t U = *n_touched;
  const int64_t per = (U + kRsBlocks - 1) / kRsBlocks;
  *lo = int64_t(blockIdx.x) * per;
  *hi = *lo + per < U ? *lo + per : U;
}

// sum of one int per thread over the block (every thread gets it)
__device__ __forceinline__ int rs_block_sum(int v, int* red) {
  v = wave_sum_i(v);
  __syncthreads();
  if ((threadIdx.x & 63) == 0) red[threadIdx.x >> 6] = v;
  __syncthreads();
  int t = 0;
#pragma unroll
  for (int w = 0; w < kRsWaves; ++w) t += red[w];
  return t;
}

__global__ __launch_bounds__(kRsThreads) void row_state_count_kernel(const int32_t* __restrict__ touched,
                                                                     const int64_t* __restrict__ n_touched,
                                                                     const int32_t* __restrict__ slot,
                                                                     const int64_t* __restrict__ n_used,
                                                                     int* __restrict__ block_new,
                                                                     int64_t* __restrict__ base) {
  __shared__ int red[kRsWaves];
  int64_t lo, hi;
  rs_range(n_touched, &lo, &hi);
  int c = 0;
  for (int64_t i = lo + threadIdx.x; i < hi; i += kRsThreads) c += slot[touched[i]] == -1 ? 1 : 0;
  c = rs_block_sum(c, red);
  if (threadIdx.x == 0) {
    block_new[blockIdx.x] = c;
    if (blockIdx.x == 0) *base = *n_used;
  }
}

__global__ __launch_bounds__(kRsThreads) void row_state_assign_kernel(const int32_t* __restrict__ touched,
                                                                      const int64_t* __restrict__ n_touched,
                                                                      int32_t* __restrict__ slot,
                                                                      const int* __restrict__ block_new,
                                                                      const int64_t* __restrict__ base,
                                                                      int64_t capacity, int64_t* __restrict__ n_used) {
  __shared__ int red[kRsWaves];
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  int before = 0;
  for (int b = threadIdx.x; b < int(blockIdx.x); b += kRsThreads) before += block_new[b];
  before = rs_block_sum(before, red);
  int64_t lo, hi;
  rs_range(n_touched, &lo, &hi);
  int64_t next = *base + before;
  for (int64_t i0 = lo; i0 < hi; i0 += kRsThreads) {  // block-uniform trip count
    const int64_t i = i0 + threadIdx.x;
    const int32_t r = i < hi ? touched[i] : 0;
    const bool isnew = i < hi && slot[r] == -1;
    int wt = 0;
    const int wr = wave_excl_scan(isnew ? 1 : 0, &wt);
    __syncthreads();
    if (lane == 0) red[wave] = wt;
    __syncthreads();
    int off = 0, tot = 0;
#pragma unroll
    for (int w = 0; w < kRsWaves; ++w) {
      off += w < wave ? red[w] : 0;
      tot += red[w];
    }
    if (isnew) {
      const int64_t sl = next + off + wr;
      if (sl < capacity) slot[r] = int32_t(-2 - sl);
    }
    next += tot;
  }
  if (blockIdx.x == kRsBlocks - 1 && threadIdx.x == 0) *n_used = *base + before + block_new[blockIdx.x];
}

}  // namespace

size_t row_state_temp_bytes() { return size_t(kRsBlocks) * sizeof(int) + 64; }

hipError_t launch_row_state_assign(hipStream_t s, const int32_t* touched, const int64_t* n_touched, int32_t* slot,
                                   int64_t capacity, int64_t* n_used, void* tmp) {
  int64_t* base = static_cast<int64_t*>(tmp);
  int* block_new = reinterpret_cast<int*>(static_cast<char*>(tmp) + 64);
  hipLaunchKernelGGL(row_state_count_kernel, dim3(kRsBlocks), dim3(kRsThreads), 0, s, touched, n_touched, slot,
                     n_used, block_new, base);
  hipLaunchKernelGGL(row_state_assign_kernel, dim3(kRsBlocks), dim3(kRsThreads), 0, s, touched, n_touched, slot,
                     block_new, base, capacity, n_used);
  return hipGetLastError();
}

size_t value_grad_aux_bytes(int64_t nitems, int d_value) {
  const int64_t slots = 2 * (nitems / kVgChunk) + 2;  // chunks of runs longer than a chunk: < 2 N / kVgChunk
  return size_t(slots) * (size_t(d_value) * 4 + 8 + 8) + 64;
}

VgPlan value_grad_plan(void* aux, int64_t nitems, int d_value) {
  const int64_t slots = 2 * (nitems / kVgChunk) + 2;
  char* ap = static_cast<char*>(aux);
  VgPlan p;
  p.counts = reinterpret_cast<uint32_t*>(ap);
  p.chunk_list = reinterpret_cast<int2*>(ap + 64 + size_t(slots) * d_value * 4);
  p.long_list = p.chunk_list + slots;
  return p;
}

hipError_t launch_value_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg,
                             int64_t nitems, const uint32_t* sorted_rows, const int32_t* sorted_c, const float* w,
                             const void* dY, const void* V, float* dV, float* dw, int R, int d_value,
                             bool accumulate, void* aux, const VgAdam* adam, bool plan_ready,
                             const VgPlan* plan_in) {
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
  a.Vout = nullptr;
  a.am = a.av = nullptr;
  a.b1 = a.b2 = a.eps = a.step_size = a.inv_sqrt_bc2 = 0.f;
  a.sgd = 0;
  a.slot = nullptr;
  a.capacity = 0;
  if (adam) {
    a.sgd = adam->sgd;
    a.slot = adam->slot;
    a.capacity = adam->capacity;
    a.Vout = adam->V;
    a.am = adam->m;
    a.av = adam->v;
    a.b1 = adam->beta1;
    a.b2 = adam->beta2;
    a.eps = adam->eps;
    a.step_size = adam->step_size;
    a.inv_sqrt_bc2 = adam->inv_sqrt_bc2;
  }
  // plan_in: a plan made elsewhere (ready); else the plan in aux
  const VgPlan plan = plan_in ? *plan_in : value_grad_plan(aux, nitems, d_value);
  a.counts = plan.counts;
  a.partial = reinterpret_cast<float*>(ap + 64);
  a.chunk_list = plan.chunk_list;
  a.long_list = plan.long_list;
  if (!plan_ready && plan_in == nullptr) {
    hipLaunchKernelGGL(zero_u32_kernel, dim3(1), dim3(64), 0, s, plan.counts, 2);
    int64_t pb = (nitems + 255) / 256;
    if (pb > 4096) pb = 4096;
    if (pb < 1) pb = 1;
    hipLaunchKernelGGL(long_run_plan_kernel, dim3(unsigned(pb)), dim3(256), 0, s, seg_start, nseg, kVgChunk,
                       static_cast<const uint32_t*>(nullptr), 0u, plan.chunk_list, plan.long_list, plan.counts);
  }
  const dim3 block(256);
  const dim3 grid_long(grid_waves(slots, 1024));
#define PKM_VG_AD(TT, NV, AD)                                                                                \
  do {                                                                                                       \
    const dim3 grid(resident_grid(reinterpret_cast<const void*>(value_grad_kernel<TT, NV, 0, AD>), nitems)); \
    hipLaunchKernelGGL((value_grad_kernel<TT, NV, 0, AD>), grid, block, 0, s, a);                            \
    hipLaunchKernelGGL((value_grad_kernel<TT, NV, 1, AD>), grid_long, block, 0, s, a);                       \
  } while (0)
#define PKM_VG(TT, NV)            \
  do {                            \
    if (adam)                     \
      PKM_VG_AD(TT, NV, true);    \
    else                          \
      PKM_VG_AD(TT, NV, false);   \
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
#undef PKM_VG_AD
  return hipGetLastError();
}

}  // namespace pkm
