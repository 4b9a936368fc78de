// Steps a3 + a4 for bf16 queries and codebooks of 257-2048 sub-keys: sub-key
// scores of each query half and the per-half top-k, with every score of a
// 64-token (32-token for codebooks above 1024) tile kept in registers.
//
//   s1[t,h,i] = q1[t,h] . C[h,i],   s2[t,h,j] = q2[t,h] . C'[h,j]
//   I1 = the k largest s1 (score desc, index asc on ties), likewise I2.
//
// ("Meta AI 可扩展内存层", sections 4.3-4.4: each half is scored against its own
// codebook as a matrix product and only its top-k survive; product-key paper
// summary, method details: q split into q1, q2, top-k search in each half.)
//
// One workgroup = 16 waves = (TM tokens, one head, one half).  Rows are
// (token, head, half); a row's key k-th is its k-th largest (score, ~index).
// With 16 waves a lane holds at most 64 scores and the kernel fits in 128
// VGPRs, so each SIMD runs four waves of the workgroup: the selection's
// dependent chains hide each other's latency better than with eight waves of
// twice the scores (two per SIMD).
//  1. The TM x dq/2 query tile goes to LDS.
//  2. MFMA 32x32x16 bf16 (fp32 accumulation): wave w owns key tiles
//     [w KT, (w+1) KT) of 32 keys and all TM tokens; the sub-keys are the first
//     operand, so lane l of a 32x32 tile holds token l % 32 and 16 of its keys.
//     Sub-key fragments come straight from L2 in a layout where one (tile,
//     16-deep step) operand is one contiguous 1 KB block.  The scores stay in
//     registers (KT * TM/32 * 16 per lane).
//  3. Bound: each lane takes 2 maxima over consecutive runs of its scores of a
//     token, so a row has 64 group maxima (16 waves x 2 lanes x 2).  The k-th largest group maximum is
//     a lower bound of the row's k-th largest score (k groups hold a score at
//     least that large), found by a bitonic sort of the 64 maxima, 16 lanes
//     per row.
//  4. Filter: scores at or above the bound (about 44 of 1024 for k = 32 on
//     random scores) are appended to the row's LDS list as (key, ~index)
//     words; an LDS counter per row hands out the slots.
//  5. The <= 64 survivors of a row are bitonic-sorted, 16 lanes per row and 4
//     words per lane; the first k are the row's list, by score descending and
//     index ascending (the words are distinct).  A row with more than 64
//     survivors (heavy ties) is listed instead, and a second launch recomputes
//     its scores (fp32 dot products, one workgroup per listed row) and takes
//     its exact k words by bisection over the 64-bit words.
#include "common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkm {

namespace {

constexpr int kSelWaves = 16;
constexpr int kSelThreads = kSelWaves * 64;
constexpr int kSelCand = 64;  // candidate slots per row
constexpr int kSelLdsLimit = 96 * 1024;

__device__ __forceinline__ f32x16 mma32(const u32x4& a, const u32x4& b, const f32x16& c) {
  return __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a), __builtin_bit_cast(bf16x8, b), c, 0,
                                                 0, 0);
}

// Packed sub-keys of both halves, [half p][head][32-key tile][16-deep step][64
// lanes] 16-byte fragments: lane l of (tile, step) holds key tile * 32 + l % 32,
// dims step * 16 + 8 (l / 32) .. +8 (zeros past the codebook's last key).
// Also clears the count of the overflow list (the scoring launch after it appends).
__global__ __launch_bounds__(256) void pack_keys32_kernel(const bf16_t* __restrict__ C, int n1,
                                                          const bf16_t* __restrict__ Cp, int n2, int heads, int half,
                                                          int ntile, int nks, u32x4* __restrict__ out,
                                                          uint32_t* __restrict__ ovf_count) {
  if (blockIdx.x == 0 && threadIdx.x == 0) *ovf_count = 0u;
  const int64_t per_half = int64_t(heads) * ntile * nks * 64;
  const int64_t total = 2 * per_half;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(gridDim.x) * 256) {
    const int p = i >= per_half ? 1 : 0;
    const int64_t j = i - p * per_half;
    const int lane = int(j & 63);
    const int64_t fr = j >> 6;
    const int ks = int(fr % nks);
    const int64_t tl = fr / nks;
    const int tile = int(tl % ntile);
    const int hh = int(tl / ntile);
    const int n = p ? n2 : n1;
    const int row = tile * 32 + (lane & 31);
    const int kk = ks * 16 + (lane >> 5) * 8;
    u32x4 v = {0, 0, 0, 0};
    if (row < n) v = ld16((p ? Cp : C) + (size_t(hh) * n + row) * half + kk);
    out[i] = v;
  }
}

// One compare-exchange of a bitonic sort, descending over the whole sequence:
// element i (this one) against i ^ stride (o); size is the merge size.
template <typename K>
__device__ __forceinline__ K bitonic_pick(K x, K o, int i, int stride, int size) {
  const bool lower = (i & stride) == 0;
  const bool desc = (i & size) == 0;
  const K mx = x > o ? x : o;
  const K mn = x > o ? o : x;
  return lower == desc ? mx : mn;
}

// Bitonic sort, descending, of 64 values per group of 16 lanes (4 tokens per
// wave), element i = 4 (lane % 16) + v held in x[v].  Strides 1 and 2 pair
// values of one lane; larger strides pair lane l with l ^ (stride / 4).
template <typename K>
__device__ __forceinline__ void sort64_16lanes(K (&x)[4], int lane) {
  const int s = lane & 15;
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      if (stride >= 4) {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          K o;
          if constexpr (sizeof(K) == 8)
            o = K(xor_lane_u64(uint64_t(x[v]), stride >> 2));
          else
            o = K(xor_lane(uint32_t(x[v]), stride >> 2));
          x[v] = bitonic_pick<K>(x[v], o, 4 * s + v, stride, size);
        }
      } else {
#pragma unroll
        for (int v = 0; v < 4; ++v) {
          if (v & stride) continue;
          const int i = 4 * s + v;
          const K a = x[v], b = x[v | stride];
          const K mx = a > b ? a : b, mn = a > b ? b : a;
          const bool desc = (i & size) == 0;
          x[v] = desc ? mx : mn;
          x[v | stride] = desc ? mn : mx;
        }
      }
    }
  }
}

template <int KT, int NT>
__global__ __launch_bounds__(kSelThreads) void score_select_kernel(
    const bf16_t* __restrict__ q, int64_t ntok, int F, int dq, int half, int qstride, const u32x4* __restrict__ P,
    int ntile, int nks, int nk, int nk2, int heads, int k, int32_t* __restrict__ sub_idx,
    float* __restrict__ sub_score, uint32_t* __restrict__ ovf_count, uint32_t* __restrict__ ovf_rows) {
  constexpr int TM = 32 * NT;
  constexpr int NV = KT * 16;  // scores per lane and token tile
  constexpr int kG = 32 / kSelWaves;  // group maxima per lane and token: 64 per row
  extern __shared__ __attribute__((aligned(16))) char smem[];
  bf16_t* qt = reinterpret_cast<bf16_t*>(smem);
  char* uni = smem + size_t(TM) * qstride * 2;                // group maxima, then candidate words
  uint32_t* gmax = reinterpret_cast<uint32_t*>(uni);          // [TM][64]
  uint64_t* cand = reinterpret_cast<uint64_t*>(uni);          // [TM][kSelCand]
  uint32_t* bound = reinterpret_cast<uint32_t*>(uni + size_t(TM) * kSelCand * 8);  // [TM]
  uint32_t* cnt = bound + TM;                                 // [TM]
  u32x2* spare = reinterpret_cast<u32x2*>(cnt + TM);          // [kSelThreads] one per lane, discarded writes

  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  // consecutive workgroups take different (head, half) pairs: the dispatcher
  // deals workgroups to the XCDs in turn, so an XCD keeps few codebooks in L2
  const int combos = heads * 2;
  const int combo = int(blockIdx.x % unsigned(combos));
  const int hh = combo >> 1, p = combo & 1;
  const int64_t t0 = int64_t(blockIdx.x / unsigned(combos)) * TM;
  const int ncols = p ? nk2 : nk;

  // the wave's first sub-key fragments are requested before the query tile
  // lands (their L2 latency overlaps the tile's)
  const u32x4* kb = P + ((size_t(p) * heads + hh) * ntile + size_t(wave) * KT) * nks * 64 + lane;
  const size_t tstride = size_t(nks) * 64;
  u32x4 a0[KT];
#pragma unroll
  for (int t = 0; t < KT; ++t) a0[t] = kb[t * tstride];

  // 1. query tile -> LDS
  {
    const int vpr = half / 8;
    const bf16_t* qsrc = q + size_t(hh) * dq + size_t(p) * half;
    for (int e = tid; e < TM * vpr; e += kSelThreads) {
      const int r = e / vpr;
      const int kk = (e - r * vpr) * 8;
      u32x4 v = {0, 0, 0, 0};
      if (t0 + r < ntok) v = ld16(qsrc + size_t(t0 + r) * F + kk);
      st16(qt + size_t(r) * qstride + kk, v);
    }
    if (tid < TM) cnt[tid] = 0;
  }
  __syncthreads();

  // 2. scores of the wave's KT key tiles x TM tokens
  f32x16 acc[KT][NT];
#pragma unroll
  for (int t = 0; t < KT; ++t)
#pragma unroll
    for (int n = 0; n < NT; ++n)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[t][n][e] = 0.f;
  {
    const bf16_t* qb = qt + size_t(lane & 31) * qstride + (lane >> 5) * 8;
    for (int ks = 0; ks < nks; ++ks) {
      u32x4 a1[KT];  // the next step's fragments, in flight during this step's MFMAs
      const int kn = ks + 1 < nks ? ks + 1 : ks;
#pragma unroll
      for (int t = 0; t < KT; ++t) a1[t] = kb[t * tstride + size_t(kn) * 64];
      u32x4 b[NT];
#pragma unroll
      for (int n = 0; n < NT; ++n) b[n] = ld16(qb + size_t(n) * 32 * qstride + ks * 16);
#pragma unroll
      for (int t = 0; t < KT; ++t)
#pragma unroll
        for (int n = 0; n < NT; ++n) acc[t][n] = mma32(a0[t], b[n], acc[t][n]);
#pragma unroll
      for (int t = 0; t < KT; ++t) a0[t] = a1[t];
    }
  }
  // lane's key of score (t, e): 32 (wave KT + t) + 8 (e / 4) + 4 (lane / 32) + e % 4
  const int colbase = wave * KT * 32 + 4 * (lane >> 5);
  // scores of keys past the codebook do not take part
  if ((wave + 1) * KT * 32 > ncols) {  // wave-uniform
#pragma unroll
    for (int t = 0; t < KT; ++t)
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int col = colbase + t * 32 + 8 * (e >> 2) + (e & 3);
#pragma unroll
        for (int n = 0; n < NT; ++n)
          if (col >= ncols) acc[t][n][e] = -INFINITY;
      }
  }

  // 3. kG group maxima per lane and token: runs of NV / kG consecutive scores
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    float g[kG];
#pragma unroll
    for (int gi = 0; gi < kG; ++gi) {
      float m = -INFINITY;
#pragma unroll
      for (int j = gi * (NV / kG); j < (gi + 1) * (NV / kG); ++j) m = fmaxf(m, acc[j / 16][n][j % 16]);
      g[gi] = m;
    }
    const int row = n * 32 + (lane & 31);
    uint32_t* gd = gmax + size_t(row) * 64 + wave * (2 * kG) + (lane >> 5) * kG;
#pragma unroll
    for (int gi = 0; gi < kG; ++gi) gd[gi] = float_key(g[gi]);
  }
  __syncthreads();

  // bound of each row: the k-th largest of its 64 group maxima (16 lanes per row)
  for (int r0 = wave * 4; r0 < TM; r0 += kSelWaves * 4) {
    const int row = r0 + (lane >> 4);
    const u32x4 w = ld16(gmax + size_t(row) * 64 + (lane & 15) * 4);
    uint32_t x[4] = {w.x, w.y, w.z, w.w};
    sort64_16lanes<uint32_t>(x, lane);
    const int src = (lane & ~15) + (k - 1) / 4;
    const int v = (k - 1) & 3;
    const uint32_t mine = v == 0 ? x[0] : v == 1 ? x[1] : v == 2 ? x[2] : x[3];
    const uint32_t kth = uint32_t(__shfl(int(mine), src, 64));
    if ((lane & 15) == 0) bound[row] = kth;
  }
  __syncthreads();

  // 4. filter: every score at or above its row's bound goes to the row's list as
  // (score bits, column); the others are written to the lane's spare slot, so the
  // loop has no branch per score.  A lane whose survivors would pass the list's
  // end (its row goes to the exact launch) sends all of them to the spare slot.
  float bf[NT];
  uint32_t slot[NT];
  bool fits[NT];
  u32x2* rowbuf[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    const int row = n * 32 + (lane & 31);
    const bool live = t0 + row < ntok;
    bf[n] = key_float(bound[row]);
    int c = 0;
#pragma unroll
    for (int j = 0; j < NV; ++j) c += acc[j / 16][n][j % 16] >= bf[n] ? 1 : 0;
    slot[n] = 0;
    if (live && c > 0) slot[n] = atomicAdd(&cnt[row], uint32_t(c));
    fits[n] = live && slot[n] + uint32_t(c) <= uint32_t(kSelCand);
    rowbuf[n] = reinterpret_cast<u32x2*>(cand + size_t(row) * kSelCand);
  }
  u32x2* mine = spare + tid;
  // the column base and the bounds again, opaque to the compiler: otherwise it
  // computes every column of the loop below right after the MFMAs, and keeps
  // the count's compare masks for the stores, all live at once.  A lane whose
  // survivors do not fit compares against NaN, which no score reaches.
  int cbf = colbase;
  asm volatile("" : "+v"(cbf));
  float bs[NT];
#pragma unroll
  for (int n = 0; n < NT; ++n) {
    bs[n] = fits[n] ? bf[n] : __builtin_nanf("");
    asm volatile("" : "+v"(bs[n]));
  }
#pragma unroll
  for (int j = 0; j < NV; ++j) {
    const uint32_t col = uint32_t(cbf + (j / 16) * 32 + 8 * ((j % 16) >> 2) + (j & 3));
#pragma unroll
    for (int n = 0; n < NT; ++n) {
      const float s = acc[j / 16][n][j % 16];
      const bool keep = s >= bs[n];
      *(keep ? rowbuf[n] + slot[n] : mine) = u32x2{__float_as_uint(s), col};
      slot[n] += keep ? 1u : 0u;
    }
  }
  __syncthreads();
  // rows with more survivors than slots go to the exact second launch
  if (tid < TM && t0 + tid < ntok && cnt[tid] > uint32_t(kSelCand))
    ovf_rows[atomicAdd(ovf_count, 1u)] = uint32_t(((t0 + tid) * heads + hh) * 2 + p);

  // 5. sort each row's words (16 lanes per row, 4 rows per wave at a time); the first k are its list
  for (int r0 = wave * 4; r0 < TM; r0 += kSelWaves * 4) {
    const int row = r0 + (lane >> 4);
    const int64_t t = t0 + row;
    const uint32_t nc = cnt[row];  // rows above kSelCand are written by the exact launch
    const u32x2* src = reinterpret_cast<const u32x2*>(cand + size_t(row) * kSelCand) + (lane & 15) * 4;
    uint64_t x[4];
#pragma unroll
    for (int v = 0; v < 4; ++v) {
      const u32x2 e = uint32_t((lane & 15) * 4 + v) < nc ? src[v] : u32x2{0u, 0u};
      x[v] = uint32_t((lane & 15) * 4 + v) < nc
                 ? (uint64_t(float_key(__uint_as_float(e.x))) << 32) | uint32_t(~e.y)
                 : 0ull;
    }
    sort64_16lanes<uint64_t>(x, lane);
    if (t < ntok && nc <= uint32_t(kSelCand)) {
      const size_t o = ((size_t(t) * heads + hh) * 2 + p) * k;
#pragma unroll
      for (int v = 0; v < 4; ++v) {
        const int i = (lane & 15) * 4 + v;
        if (i < k) {
          sub_idx[o + i] = int32_t(~uint32_t(x[v]));
          sub_score[o + i] = key_float(uint32_t(x[v] >> 32));
        }
      }
    }
  }
}

// The listed rows (token, head, half as ((t heads + h) 2 + p)), one workgroup
// each.  The row's scores are recomputed as fp32 dot products: a group of 16
// lanes takes one sub-key, each lane 8-dim pieces of it (coalesced 16-byte
// loads; eight sub-keys per group and two pieces of each in flight), and the
// group's partial sums are added with lane exchanges.  Then the k largest (key, ~index) words come from
// a bisection over the 64-bit words, every thread holding up to four of them
// (the words are distinct, so exactly k are at or above the result), and are
// sorted by one wave.
constexpr int kExactThreads = 512;
constexpr int kExactSlots = kExactThreads / 16;  // sub-keys per round and column of 16-lane groups
constexpr int kExactU = 8;                       // sub-keys per group in flight
constexpr int kExactWords = 2048 / kExactThreads;

__global__ __launch_bounds__(kExactThreads) void score_rows_exact_kernel(
    const bf16_t* __restrict__ q, int F, int dq, int half, const bf16_t* __restrict__ C,
    const bf16_t* __restrict__ Cp, int nk, int nk2, int heads, int k, const uint32_t* __restrict__ count,
    const uint32_t* __restrict__ rows, int32_t* __restrict__ sub_idx, float* __restrict__ sub_score) {
  __shared__ float qs[512];
  __shared__ float sc[2048];
  __shared__ uint32_t wc[2][kExactThreads / 64];
  __shared__ uint32_t nsel;
  __shared__ uint64_t top[64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  const int g = lane & 15;
  const int slot = wave * 4 + (lane >> 4);
  const uint32_t n = *count;
  for (uint32_t it = blockIdx.x; it < n; it += gridDim.x) {
    const uint32_t r = rows[it];
    const int p = int(r & 1u);
    const int hh = int((r >> 1) % uint32_t(heads));
    const int64_t t = int64_t(r / (2u * uint32_t(heads)));
    const int ncols = p ? nk2 : nk;
    const bf16_t* K = (p ? Cp : C) + size_t(hh) * ncols * half;
    for (int d = tid; d < half; d += kExactThreads)
      qs[d] = to_f32<bf16_t>(q[size_t(t) * F + size_t(hh) * dq + size_t(p) * half + d]);
    if (tid == 0) nsel = 0u;
    __syncthreads();
    const int nch = half / 8;
    for (int j0 = 0; j0 < ncols; j0 += kExactSlots * kExactU) {
      float acc[kExactU];
#pragma unroll
      for (int u = 0; u < kExactU; ++u) acc[u] = 0.f;
      for (int c0 = g; c0 < nch; c0 += 32) {  // two 8-dim pieces per lane and sub-key in flight
        u32x4 v[2][kExactU];
#pragma unroll
        for (int hp = 0; hp < 2; ++hp)
#pragma unroll
          for (int u = 0; u < kExactU; ++u) {
            const int j = j0 + u * kExactSlots + slot, c = c0 + 16 * hp;
            v[hp][u] = j < ncols && c < nch ? ld16(K + size_t(j) * half + c * 8) : u32x4{0u, 0u, 0u, 0u};
          }
#pragma unroll
        for (int hp = 0; hp < 2; ++hp) {
          const int c = c0 + 16 * hp;
          if (c >= nch) continue;
          float qv[8];
#pragma unroll
          for (int e = 0; e < 8; ++e) qv[e] = qs[c * 8 + e];
#pragma unroll
          for (int u = 0; u < kExactU; ++u) {
            const uint32_t wd[4] = {v[hp][u].x, v[hp][u].y, v[hp][u].z, v[hp][u].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
              acc[u] = fmaf(qv[2 * e], __uint_as_float(wd[e] << 16), acc[u]);
              acc[u] = fmaf(qv[2 * e + 1], __uint_as_float(wd[e] & 0xFFFF0000u), acc[u]);
            }
          }
        }
      }
#pragma unroll
      for (int u = 0; u < kExactU; ++u) {
#pragma unroll
        for (int m = 8; m >= 1; m >>= 1) acc[u] += __shfl_xor(acc[u], m, 64);
        const int j = j0 + u * kExactSlots + slot;
        if (g == 0 && j < ncols) sc[j] = acc[u];
      }
    }
    __syncthreads();
    uint64_t w[kExactWords];
#pragma unroll
    for (int v = 0; v < kExactWords; ++v) {
      const int j = tid + v * kExactThreads;
      w[v] = j < ncols ? (uint64_t(float_key(sc[j])) << 32) | uint32_t(~uint32_t(j)) : 0ull;
    }
    uint64_t res = 0;
    for (int b = 63; b >= 0; --b) {
      const uint64_t cand = res | (uint64_t(1) << b);
      uint32_t c = 0;
#pragma unroll
      for (int v = 0; v < kExactWords; ++v) c += uint32_t(popc64(ballot(w[v] >= cand)));
      if (lane == 0) wc[b & 1][wave] = c;
      __syncthreads();
      uint32_t tot = 0;
#pragma unroll
      for (int x = 0; x < kExactThreads / 64; ++x) tot += wc[b & 1][x];
      if (tot >= uint32_t(k)) res = cand;
    }
#pragma unroll
    for (int v = 0; v < kExactWords; ++v)
      if (w[v] >= res) top[atomicAdd(&nsel, 1u)] = w[v];
    __syncthreads();
    if (wave == 0) {
      uint64_t x = lane < k ? top[lane] : 0ull;
      x = wave_sort_desc_u64(x);
      if (lane < k) {
        const size_t o = ((size_t(t) * heads + hh) * 2 + p) * k + lane;
        sub_idx[o] = int32_t(~uint32_t(x));
        sub_score[o] = key_float(uint32_t(x >> 32));
      }
    }
    __syncthreads();
  }
}

struct SelPlan {
  int KT, NT, ntile, nks, qstride;
  size_t lds;
};

SelPlan sel_plan(int half, int nk, int nk2) {
  SelPlan s{};
  const int nmax = nk > nk2 ? nk : nk2;
  s.KT = (nmax <= 512 ? 16 : nmax <= 1024 ? 32 : 64) / kSelWaves;
  s.NT = nmax > 1024 ? 1 : 2;
  s.ntile = kSelWaves * s.KT;
  s.nks = half / 16;
  s.qstride = half + 8;
  const int TM = 32 * s.NT;
  s.lds = size_t(TM) * s.qstride * 2 + size_t(TM) * kSelCand * 8 + size_t(TM) * 8 + size_t(kSelThreads) * 8;
  return s;
}

}  // namespace

bool score_select_supported(int dtype, int half, int nk, int nk2, int k, bool idw) {
  if (dtype != kBF16 || idw || k < 1 || k > 32) return false;
  if (half % 16 || half < 16) return false;
  const int nmax = nk > nk2 ? nk : nk2, nmin = nk < nk2 ? nk : nk2;
  if (nmax <= 256 || nmax > 2048) return false;
  const SelPlan s = sel_plan(half, nk, nk2);
  if (half > (s.NT == 2 ? 256 : 512)) return false;
  // every group of scores must hold keys of the codebook for the bound to be useful:
  // the smaller codebook fills more than half of the padded tiles
  return 2 * nmin > s.ntile * 32 && s.lds <= kSelLdsLimit;
}

size_t score_select_packed_bytes(int heads, int half, int nk, int nk2) {
  const SelPlan s = sel_plan(half, nk, nk2);
  return size_t(2) * heads * s.ntile * s.nks * 64 * 16;
}

size_t score_select_list_bytes(int64_t ntok, int heads) { return 256 + size_t(ntok) * heads * 2 * 4; }

hipError_t launch_score_select(hipStream_t s, const void* q, int64_t ntok, int heads, int dq, const void* C,
                               const void* Cp, int nk, int nk2, int k, int32_t* sub_idx, float* sub_score,
                               void* packed, void* list) {
  const int half = dq / 2;
  if (!score_select_supported(kBF16, half, nk, nk2, k, false)) return hipErrorInvalidValue;
  const SelPlan pl = sel_plan(half, nk, nk2);
  u32x4* P = static_cast<u32x4*>(packed);
  const int64_t total = int64_t(2) * heads * pl.ntile * pl.nks * 64;
  int64_t pb = (total + 255) / 256;
  if (pb > 4096) pb = 4096;
  uint32_t* ovf_count = static_cast<uint32_t*>(list);
  uint32_t* ovf_rows = ovf_count + 64;
  hipLaunchKernelGGL(pack_keys32_kernel, dim3(unsigned(pb)), dim3(256), 0, s, static_cast<const bf16_t*>(C), nk,
                     static_cast<const bf16_t*>(Cp), nk2, heads, half, pl.ntile, pl.nks, P, ovf_count);
  const int TM = 32 * pl.NT;
  const int64_t tiles = (ntok + TM - 1) / TM;
  const dim3 grid(unsigned(tiles * heads * 2));
  const int F = heads * dq;
  if (ntok == 0) return hipGetLastError();
#define PKM_SEL_CASE(KTV, NTV)                                                                                  \
  if (pl.KT == KTV) {                                                                                           \
    static LdsLimit lim; /* the largest plan's LDS, set once per device */                                      \
    const hipError_t e = lim.ensure(reinterpret_cast<const void*>(score_select_kernel<KTV, NTV>), kSelLdsLimit); \
    if (e != hipSuccess) return e;                                                                              \
    hipLaunchKernelGGL((score_select_kernel<KTV, NTV>), grid, dim3(kSelThreads), pl.lds, s,                      \
                       static_cast<const bf16_t*>(q), ntok, F, dq, half, pl.qstride, P, pl.ntile, pl.nks, nk, nk2, \
                       heads, k, sub_idx, sub_score, ovf_count, ovf_rows);                                      \
  }
  PKM_SEL_CASE(1, 2)
  PKM_SEL_CASE(2, 2)
  PKM_SEL_CASE(4, 1)
#undef PKM_SEL_CASE
  // rows with heavy ties (usually none): exact selection, one workgroup per listed row
  hipLaunchKernelGGL(score_rows_exact_kernel, dim3(256), dim3(kExactThreads), 0, s, static_cast<const bf16_t*>(q), F, dq, half,
                     static_cast<const bf16_t*>(C), static_cast<const bf16_t*>(Cp), nk, nk2, heads, k, ovf_count,
                     ovf_rows, sub_idx, sub_score);
  return hipGetLastError();
}

}  // namespace pkm
