// Steps a3 + a4: sub-key scores of each query half and the per-half top-k.
//
//   s1[t,h,i] = q1[t,h] . C[h,i],   s2[t,h,j] = q2[t,h] . C'[h,j]
//   I1 = the k largest s1 (score desc, index asc on ties), likewise I2.
//
// ("Meta AI 可扩展内存层", sections 4.3-4.4: each half is scored against its own
// codebook as a matrix product and only its top-k survive; product-key paper
// summary, method details: q split into q1, q2, top-k search in each half.)
//
// One workgroup = 8 waves = (TM tokens, one head, one half).
//  1. The TM x dq/2 query tile is staged in LDS.
//  2. MFMA (bf16 16x16x32 or fp32 16x16x4, fp32 accumulation): each wave owns
//     16-column tiles of the TM x |C| score tile and streams its sub-key rows
//     from L2 (the codebooks are small); the scores land in LDS and never
//     reach HBM.  The sub-keys are first repacked so that the 64 lane
//     fragments of one (16-key tile, k step) operand are one contiguous 1 KB
//     block: the operand read in MFMA order would touch 16 half-used cache
//     lines per instruction, which the texture path serves at about a third
//     of the rate of a contiguous read.
//  3. Selection: each wave owns TM/8 rows and works on them together (their
//     dependency chains overlap).  A lane holds |C|/64 scores of a row; the
//     k-th largest of the 64 lane maxima (bisection on order-preserving keys,
//     with ballots) is a lower bound of the row's k-th largest score, so every
//     score below it is dropped by a plain float compare; the <= 64 survivors
//     are compacted (DPP prefix sum) into the row's own LDS slot and
//     bitonic-sorted as (key, ~index) 64-bit words, which orders them by score
//     and then lowest index.  Rows where more than 64 scores pass the bound
//     (heavy ties) take an exact bisection over all scores instead.
#include "common.h"
#include "kernels.h"
#include "lane_ops.h"

namespace pkm {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = kWaves * 64;
constexpr size_t kLdsLimit = 160 * 1024;

__device__ __forceinline__ void wave_lds_sync() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
  __builtin_amdgcn_wave_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
}

// Wave-wide maximum / minimum, the result in every lane (xor butterfly).
__device__ __forceinline__ float wave_max_f32(float v) {
#pragma unroll
  for (int st = 1; st < 64; st <<= 1) v = fmaxf(v, __uint_as_float(xor_lane(__float_as_uint(v), st)));
  return v;
}
__device__ __forceinline__ float wave_min_f32(float v) {
#pragma unroll
  for (int st = 1; st < 64; st <<= 1) v = fminf(v, __uint_as_float(xor_lane(__float_as_uint(v), st)));
  return v;
}

constexpr int kBoundSteps = 12;       // halvings of the selection bound's search range
constexpr float kIdwFloor = 1e-12f;  // squared-distance floor of the IDW scores

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

template <typename T>
struct ScoreTraits;
template <>
struct ScoreTraits<bf16_t> {
  static constexpr int VE = 8;   // elements per 16-byte lane vector
  static constexpr int KC = 32;  // k covered by one 16-byte vector per lane (4 lane groups)
  __device__ __forceinline__ static f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct ScoreTraits<float> {
  static constexpr int VE = 4;
  static constexpr int KC = 16;
  __device__ __forceinline__ static f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    // Lane group g holds k = 4g..4g+3 of this 16-wide slice for both operands;
    // MFMA step e consumes element e, so the 4 steps cover all 16 k.
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};


// Exclusive prefix sum of one int per lane (DPP row shifts inside rows of 16,
// then row broadcasts across rows); *total gets the wave total.
__device__ __forceinline__ int wave_excl_scan_dpp(int v, int* total) {
  int x = v;
  const int lane = lane_id();
  int y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x111, 0xF, 0xF, false);  // row_shr:1
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x112, 0xF, 0xF, false);  // row_shr:2
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x114, 0xF, 0xF, false);  // row_shr:4
  x += y;
  y = __builtin_amdgcn_update_dpp(0, x, 0x118, 0xF, 0xF, false);  // row_shr:8
  x += y;
  // inclusive within rows of 16; add the totals of earlier rows
  const int r0 = __builtin_amdgcn_readlane(x, 15), r1 = __builtin_amdgcn_readlane(x, 31),
            r2 = __builtin_amdgcn_readlane(x, 47), r3 = __builtin_amdgcn_readlane(x, 63);
  const int row = lane >> 4;
  x += (row > 0 ? r0 : 0) + (row > 1 ? r1 : 0) + (row > 2 ? r2 : 0);
  *total = r0 + r1 + r2 + r3;
  return x - v;
}

// Bitonic sort, descending, of N independent uint64 values per lane across the wave.
template <int N>
__device__ __forceinline__ void wave_sort_desc_u64_n(uint64_t* v) {
  const int lane = lane_id();
#pragma unroll
  for (int size = 2; size <= 64; size <<= 1) {
#pragma unroll
    for (int stride = size >> 1; stride > 0; stride >>= 1) {
      const bool take_max = ((lane & stride) == 0) == ((lane & size) == 0);
#pragma unroll
      for (int q = 0; q < N; ++q) {
        const uint64_t o = xor_lane_u64(v[q], stride);
        const bool gt = v[q] > o;
        v[q] = (gt == take_max) ? v[q] : o;
      }
    }
  }
}

// Column of a row's j-th value in a lane: 16-byte runs of 4 consecutive
// columns per lane when a lane holds at least 4 values (one ds_read_b128 per
// run), else one column per 64.
template <int NPL>
__device__ __forceinline__ int col_of(int j, int lane) {
  return NPL >= 4 ? 256 * (j >> 2) + 4 * lane + (j & 3) : j * 64 + lane;
}

// Exact top-k of one row held as NPL scores per lane (column col0 +
// col_of(j, lane)), written as (key, ~column) words into slot[0..k): the
// words are distinct, so the k-th largest word (bisection over all 64 bits,
// counts by ballot) splits off exactly the k best, ties going to the lowest
// column.  The fallback for rows where heavy ties defeat the cheap bound.
template <int NPL>
__device__ __forceinline__ void exact_topk(const float* v, int k, int lane, uint32_t col0, uint64_t* slot) {
  uint64_t key[NPL];
#pragma unroll
  for (int j = 0; j < NPL; ++j)
    key[j] = v[j] == -INFINITY ? 0ull
                               : (uint64_t(float_key(v[j])) << 32) | uint32_t(~(col0 + uint32_t(col_of<NPL>(j, lane))));
  uint64_t res = 0;
  for (int b = 63; b >= 0; --b) {
    const uint64_t cand = res | (1ull << b);
    int c = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) c += popc64(ballot(key[j] >= cand));
    if (c >= k) res = cand;
  }
  int mine = 0;
#pragma unroll
  for (int j = 0; j < NPL; ++j) mine += key[j] >= res;
  int tot;
  int pos = wave_excl_scan(mine, &tot);
#pragma unroll
  for (int j = 0; j < NPL; ++j)
    if (key[j] >= res) slot[pos++] = key[j];
}

struct Plan {
  int TM;
  int half_pad;
  int qstride;  // elements
  int cw;       // columns per chunk (multiple of 64); rows wider than this are done chunk by chunk
  int sstride;  // floats
  int npl;
  size_t lds;
};

inline int round_up(int a, int b) { return (a + b - 1) / b * b; }

constexpr int kMaxChunk = 1024;

// Widest chunk first (one selection per row and chunk), then the tallest tile
// (a sub-key row read from L2 serves TM queries).
// Row tiles: the tallest that fits, at least 32 rows for chunks wider than 256
// columns (32 rows share each sub-key operand between two MFMA row tiles).
// small_tiles: a launch with too few 32-row tiles to fill the chip takes
// 16-row tiles (twice the blocks, each with half the work).
Plan make_plan(int dtype, int half, int ncols, bool small_tiles = false) {
  Plan p{};
  const int VE = dtype == kBF16 ? 8 : 4;
  const int KC = dtype == kBF16 ? 32 : 16;
  const int e = dtype == kBF16 ? 2 : 4;
  p.half_pad = round_up(half, KC);
  p.qstride = p.half_pad + VE;
  p.TM = 0;
  const int full = round_up(ncols, 64);
  for (int cw = full < kMaxChunk ? full : kMaxChunk; cw >= 64 && p.TM == 0; cw = round_up(cw / 2, 64)) {
    int npl = 1;
    while (npl * 64 < cw) npl *= 2;
    // a row's slot also takes the compacted (score, column) pairs: 64 of them,
    // plus 64 spare entries when a lane holds >= 4 values (>= 128 / 256 floats)
    const int smin = npl >= 4 ? 256 : 128;
    const int sstride = (cw > smin ? cw : smin) + 4;
    for (int tm = small_tiles ? 16 : 64; tm >= 16; tm /= 2) {
      const size_t lds = size_t(tm) * p.qstride * e + size_t(tm) * sstride * 4;
      if (lds <= kLdsLimit && (tm / kWaves) * npl <= 64 && tm >= (cw > 256 && !small_tiles ? 32 : 16)) {
        p.TM = tm;
        p.cw = cw;
        p.npl = npl;
        p.sstride = sstride;
        p.lds = lds;
        break;
      }
    }
    if (cw == 64) break;
  }
  if (p.TM == 0) {  // small tiles as a last resort
    const int cw = full < 256 ? full : 256;
    int npl = 1;
    while (npl * 64 < cw) npl *= 2;
    const int smin = npl >= 4 ? 256 : 128;
    const int sstride = (cw > smin ? cw : smin) + 4;
    const size_t lds = size_t(16) * p.qstride * e + size_t(16) * sstride * 4;
    if (lds <= kLdsLimit) {
      p.TM = 16;
      p.cw = cw;
      p.npl = npl;
      p.sstride = sstride;
      p.lds = lds;
    }
  }
  return p;
}

// Top-k of the union of two lists held one word per lane, each sorted
// descending in lanes 0..31 (lanes 32..63 of a are zero): the lane-wise maximum
// of a and reversed b is a bitonic sequence holding the 32 largest words of
// both, which five half-cleaner steps sort.
__device__ __forceinline__ uint64_t merge_top32(uint64_t a, uint64_t b, int lane) {
  const int src = lane < 32 ? 31 - lane : lane;
  const uint64_t br = (uint64_t(uint32_t(__shfl(int(uint32_t(b >> 32)), src, 64))) << 32) |
                      uint32_t(__shfl(int(uint32_t(b)), src, 64));
  uint64_t x = lane < 32 ? (a > br ? a : br) : 0ull;
#pragma unroll
  for (int stride = 16; stride > 0; stride >>= 1) {
    const uint64_t o = xor_lane_u64(x, stride);
    const bool take_max = (lane & stride) == 0;
    const bool gt = x > o;
    x = (gt == take_max) ? x : o;
  }
  return x;
}

// Packed operand layout, per codebook: [h][ceil(n/16) tiles][ksteps][64 lanes]
// 16-byte fragments; lane (r, g) of (tile, kstep) holds row tile*16 + r,
// elements kstep*KC + g*VE .. +VE (zeros past the last row or element).  The
// packed C' follows the packed C in memory, so one index space covers both.
//
// For the IDW scores (norms != null) the blocks from pack_blocks on compute
// |c|^2 of every sub-key row instead: C's rows, then C''s, into norms[] in
// that order.  One wave per row; lane l squares the 16-byte vectors l, l + 64,
// ... of the row, and a DPP reduction adds the lanes in a fixed order (the
// result does not change from run to run).
template <typename T>
__global__ __launch_bounds__(256) void pack_keys_kernel(const T* __restrict__ C, int n1, const T* __restrict__ Cp,
                                                        int n2, int heads, int half, int nks, int pack_blocks,
                                                        u32x4* __restrict__ out, float* __restrict__ norms) {
  using TR = ScoreTraits<T>;
  if (int(blockIdx.x) >= pack_blocks) {  // block-uniform
    constexpr int VE = Vec16<T>::N;
    const int lane = lane_id();
    const int vpr = half / VE;
    const int64_t rows1 = int64_t(heads) * n1, rows = rows1 + int64_t(heads) * n2;
    const int64_t nw = int64_t(gridDim.x - pack_blocks) * 4;
    for (int64_t r = int64_t(blockIdx.x - pack_blocks) * 4 + (threadIdx.x >> 6); r < rows; r += nw) {
      const T* c = r < rows1 ? C + size_t(r) * half : Cp + size_t(r - rows1) * half;
      float a = 0.f;
      for (int v = lane; v < vpr; v += 64) {
        float x[VE];
        Vec16<T>::widen(ld16(c + size_t(v) * VE), x);
#pragma unroll
        for (int e = 0; e < VE; ++e) a = fmaf(x[e], x[e], a);
      }
      a = wave_sum_dpp(a);
      if (lane == 0) norms[r] = a;
    }
    return;
  }
  const int64_t total1 = int64_t(heads) * ((n1 + 15) / 16) * nks * 64;
  const int64_t total = total1 + int64_t(heads) * ((n2 + 15) / 16) * nks * 64;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < total; i += int64_t(pack_blocks) * 256) {
    const bool second = i >= total1;
    const T* src = second ? Cp : C;
    const int n = second ? n2 : n1;
    const int64_t j = second ? i - total1 : i;
    const int ntile = (n + 15) / 16;
    const int lane = int(j & 63);
    const int64_t fr = j >> 6;
    const int ks = int(fr % nks);
    const int64_t tl = fr / nks;
    const int tile = int(tl % ntile);
    const int hh = int(tl / ntile);
    const int row = tile * 16 + (lane & 15);
    const int kk = ks * TR::KC + (lane >> 4) * TR::VE;
    u32x4 v = {0, 0, 0, 0};
    if (row < n && kk < half) v = ld16(src + (size_t(hh) * n + row) * half + kk);
    out[i] = v;
  }
}

// Top-k of one score chunk for RPW rows of S (rows row0, row0 + rstep, ...),
// merged into the running lists run[] (cb == 0: the chunk starts the row).
// Columns [0, cwe) of each row hold the scores of columns cb + c; each row's
// slot is reused as compaction scratch.  Selection: the k-th largest lane
// maximum (a lower bound of the row's k-th largest score, bisection on
// order-preserving keys with ballots) drops most scores by a float compare;
// the <= 64 survivors are compacted and bitonic-sorted as (key, ~column) words;
// rows with more survivors (heavy ties) take the exact path.  The rows are
// worked on together so that their latency chains overlap.
template <int NPL, int RPW>
__device__ __forceinline__ void select_chunk(float* S, int sstride, int row0, int rstep, int cwe, int cb, int k,
                                             int lane, uint64_t* run) {
  float v[RPW][NPL];
  float lmax[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const float* srow = S + size_t(row0 + q * rstep) * sstride;
    lmax[q] = -INFINITY;
    if constexpr (NPL >= 4) {
#pragma unroll
      for (int jj = 0; jj < NPL / 4; ++jj) {
        const int c0 = 256 * jj + 4 * lane;  // a run starting below cwe ends inside the row (sstride >= cw + 4)
        f32x4 t = {-INFINITY, -INFINITY, -INFINITY, -INFINITY};
        if (c0 < cwe) t = *reinterpret_cast<const f32x4*>(srow + c0);
#pragma unroll
        for (int e = 0; e < 4; ++e) v[q][4 * jj + e] = c0 + e < cwe ? t[e] : -INFINITY;
      }
    } else {
#pragma unroll
      for (int j = 0; j < NPL; ++j) {
        const int col = j * 64 + lane;
        v[q][j] = col < cwe ? srow[col] : -INFINITY;
      }
    }
#pragma unroll
    for (int j = 0; j < NPL; ++j) lmax[q] = fmaxf(lmax[q], v[q][j]);
  }
  // A lower bound of the row's k-th largest score: any value b with at least k
  // lane maxima >= b (k distinct lanes then hold a score >= b).  Bisection on
  // the value between the smallest and the largest finite lane maximum keeps
  // that invariant at the low end; kBoundSteps halvings leave the bound within
  // 1/4096 of that range below the k-th largest lane maximum, which lets a few
  // more scores through than the exact value would at a third of the
  // dependent ballot steps.  With fewer than k finite lane maxima the bound is
  // -inf (every score survives and the row takes the exact path).
  const int kc_ = k < cwe ? k : cwe;  // a chunk narrower than k keeps all its columns
  float lo[RPW], hi[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    hi[q] = wave_max_f32(lmax[q]);
    lo[q] = wave_min_f32(lmax[q] == -INFINITY ? INFINITY : lmax[q]);
  }
  bool few[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) few[q] = popc64(ballot(lmax[q] != -INFINITY)) < kc_;
#pragma unroll
  for (int it = 0; it < kBoundSteps; ++it) {
#pragma unroll
    for (int q = 0; q < RPW; ++q) {
      const float mid = lo[q] + (hi[q] - lo[q]) * 0.5f;
      const bool ok = popc64(ballot(lmax[q] >= mid)) >= kc_;
      lo[q] = ok ? mid : lo[q];
      hi[q] = ok ? hi[q] : mid;
    }
  }
  float thrv[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) thrv[q] = few[q] ? -INFINITY : lo[q];
  int cnt[RPW], total[RPW], pos[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const float thr = thrv[q];
    cnt[q] = 0;
#pragma unroll
    for (int j = 0; j < NPL; ++j) cnt[q] += v[q][j] >= thr;
    pos[q] = wave_excl_scan_dpp(cnt[q], &total[q]);
  }
  // compaction into the row's own LDS slot (its scores are in registers now)
  // as (score bits, column) pairs; rows with more than 64 survivors (heavy
  // ties) take the exact path, which writes finished (key, ~column) words
  __builtin_amdgcn_wave_barrier();
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const float thr = thrv[q];
    if (total[q] <= 64) {
      u32x2* slot = reinterpret_cast<u32x2*>(S + size_t(row0 + q * rstep) * sstride);
      if constexpr (NPL >= 4) {
        // every value is stored: survivors at their rank, the rest into the
        // lane's own spare entry 64 + lane (no per-value branch)
#pragma unroll
        for (int j = 0; j < NPL; ++j) {
          const bool keep = v[q][j] >= thr;
          slot[keep ? pos[q] : 64 + lane] = u32x2{__float_as_uint(v[q][j]), uint32_t(col_of<NPL>(j, lane))};
          pos[q] += keep ? 1 : 0;
        }
      } else {
#pragma unroll
        for (int j = 0; j < NPL; ++j)
          if (v[q][j] >= thr) slot[pos[q]++] = u32x2{__float_as_uint(v[q][j]), uint32_t(col_of<NPL>(j, lane))};
      }
    } else {
      exact_topk<NPL>(v[q], kc_, lane, uint32_t(cb), reinterpret_cast<uint64_t*>(S + size_t(row0 + q * rstep) * sstride));
    }
  }
  wave_lds_sync();
  uint64_t key[RPW];
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const u32x2* slot = reinterpret_cast<const u32x2*>(S + size_t(row0 + q * rstep) * sstride);
    if (total[q] <= 64) {
      const u32x2 e = lane < total[q] ? slot[lane] : u32x2{0u, 0u};
      key[q] = lane < total[q]
                   ? (uint64_t(float_key(__uint_as_float(e.x))) << 32) | uint32_t(~(uint32_t(cb) + e.y))
                   : 0ull;
    } else {
      key[q] = lane < kc_ ? reinterpret_cast<const uint64_t*>(slot)[lane] : 0ull;
    }
  }
  wave_sort_desc_u64_n<RPW>(key);
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    // the chunk's 32 largest words contain its top k (k <= 32)
    const uint64_t top = lane < 32 ? key[q] : 0ull;
    run[q] = cb == 0 ? top : merge_top32(run[q], top, lane);
  }
}

template <typename T, int TM, int NPL>
__global__ __launch_bounds__(kThreads) void score_topk_kernel(
    const T* __restrict__ q, int64_t ntok, int F, int dq, int half, int half_pad, int qstride,
    const u32x4* __restrict__ P1, const u32x4* __restrict__ P2, int nk, int nk2, int k, int cw, int sstride,
    int32_t* __restrict__ sub_idx, float* __restrict__ sub_score, const float* __restrict__ cc1,
    const float* __restrict__ cc2) {
  using TR = ScoreTraits<T>;
  constexpr int VE = TR::VE;
  constexpr int KC = TR::KC;
  constexpr int RT = TM / 16;
  constexpr int CT = TM >= 32 ? 256 / TM : 8;  // column tiles per pass: RT*CT*4 <= 64 accumulator registers

  extern __shared__ __attribute__((aligned(16))) char smem[];
  T* qt = reinterpret_cast<T*>(smem);
  float* S = reinterpret_cast<float*>(smem + size_t(TM) * qstride * sizeof(T));

  const int tid = threadIdx.x;
  const int wave = tid >> 6;
  const int lane = tid & 63;
  const int hh = blockIdx.y;
  const int p = blockIdx.z;
  const int heads = gridDim.y;
  const int ncols = p ? nk2 : nk;
  const int ntile = (ncols + 15) / 16;
  const int nks = half_pad / KC;
  const u32x4* keys = (p ? P2 : P1) + size_t(hh) * ntile * nks * 64;
  // IDW scores (cc1 != null): |c|^2 of this head's sub-keys; the tile then
  // holds 2 q.c - |c|^2, which orders like -|q - c|^2 (|q|^2 is one per row)
  const float* ccp = cc1 ? (p ? cc2 : cc1) + size_t(hh) * ncols : nullptr;
  const int64_t t0 = int64_t(blockIdx.x) * TM;

  // 1. query tile -> LDS (zero rows past the last token and k past dq/2)
  {
    const int vpr = half_pad / VE;
    const T* qsrc = q + size_t(hh) * dq + size_t(p) * half;
    for (int e = tid; e < TM * vpr; e += kThreads) {
      const int r = e / vpr;
      const int kk = (e - r * vpr) * VE;
      u32x4 v = {0, 0, 0, 0};
      if (t0 + r < ntok && kk < half) v = ld16(qsrc + size_t(t0 + r) * F + kk);
      st16(qt + size_t(r) * qstride + kk, v);
    }
  }
  __syncthreads();

  constexpr int RPW = TM / kWaves;
  uint64_t run[RPW];  // running top-k of the chunks done so far (lanes 0..31, descending)
  const int lrow = lane & 15;
  const int lgrp = lane >> 4;
  for (int cb = 0; cb < ncols; cb += cw) {
    const int cwe = ncols - cb < cw ? ncols - cb : cw;  // columns in this chunk

    // 2. scores of the chunk -> LDS
    const int nct = (cwe + 15) / 16;
    for (int g0 = wave * CT; g0 < nct; g0 += kWaves * CT) {
      f32x4 acc[RT][CT];
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c) acc[rt][c] = f32x4{0.f, 0.f, 0.f, 0.f};

      // this wave's tiles; tiles past the chunk are clamped (their columns are never stored)
      const u32x4* kb[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) {
        int tile = cb / 16 + g0 + c;
        tile = tile < ntile ? tile : ntile - 1;
        kb[c] = keys + size_t(tile) * nks * 64 + lane;
      }
      u32x4 bcur[CT];
#pragma unroll
      for (int c = 0; c < CT; ++c) bcur[c] = kb[c][0];
      for (int ks = 0; ks < nks; ++ks) {
        u32x4 bnext[CT];
        const int kn = ks + 1 < nks ? ks + 1 : ks;
#pragma unroll
        for (int c = 0; c < CT; ++c) bnext[c] = kb[c][size_t(kn) * 64];
        u32x4 a[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) a[rt] = ld16(qt + size_t(rt * 16 + lrow) * qstride + ks * KC + lgrp * VE);
#pragma unroll
        for (int c = 0; c < CT; ++c)
#pragma unroll
          for (int rt = 0; rt < RT; ++rt) acc[rt][c] = TR::mma(bcur[c], a[rt], acc[rt][c]);
#pragma unroll
        for (int c = 0; c < CT; ++c) bcur[c] = bnext[c];
      }
      // The sub-keys are the MFMA's first operand, so the 16x16 tile is
      // D[key][token]: lane l holds token l%16 and keys 4*(l/16)+i, i.e. four
      // consecutive scores of one query row, stored with one 16-byte write.
#pragma unroll
      for (int rt = 0; rt < RT; ++rt)
#pragma unroll
        for (int c = 0; c < CT; ++c) {
          if (g0 + c < nct) {
            f32x4 v = acc[rt][c];
            if (ccp) {  // wave-uniform
              const int key0 = cb + (g0 + c) * 16 + lgrp * 4;
#pragma unroll
              for (int i = 0; i < 4; ++i) v[i] = fmaf(2.f, v[i], -(key0 + i < ncols ? ccp[key0 + i] : 0.f));
            }
            *reinterpret_cast<f32x4*>(S + size_t(rt * 16 + lrow) * sstride + (g0 + c) * 16 + lgrp * 4) = v;
          }
        }
    }
    __syncthreads();

    // 3. per-row top-k of the chunk; wave w owns rows w, w+8, ...
    select_chunk<NPL, RPW>(S, sstride, wave, kWaves, cwe, cb, k, lane, run);
    __syncthreads();  // the next chunk's scores overwrite S
  }
  float qq[RPW];  // |q half|^2 of the wave's rows (IDW only)
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    qq[q] = 0.f;
    if (ccp) {
      const T* qr = qt + size_t(q * kWaves + wave) * qstride;
      float a = 0.f;
      for (int e = lane; e < half_pad; e += 64) {
        const float x = to_f32<T>(qr[e]);
        a = fmaf(x, x, a);
      }
      qq[q] = wave_sum_dpp(a);
    }
  }
#pragma unroll
  for (int q = 0; q < RPW; ++q) {
    const int64_t t = t0 + q * kWaves + wave;
    if (lane < k && t < ntok) {
      const size_t o = ((size_t(t) * heads + hh) * 2 + p) * k + lane;
      sub_idx[o] = int32_t(~uint32_t(run[q]));
      const float v = key_float(uint32_t(run[q] >> 32));
      // IDW: -log |q - c| = -1/2 log(|q|^2 - (2 q.c - |c|^2)), squared distance floored
      sub_score[o] = ccp ? -0.5f * logf(fmaxf(qq[q] - v, kIdwFloor)) : v;
    }
  }
}


template <typename T, int TM>
hipError_t launch_tm(hipStream_t s, const Plan& pl, const void* q, int64_t ntok, int heads, int dq, const u32x4* C,
               const u32x4* Cp, int nk, int nk2, int k, int32_t* sub_idx, float* sub_score, const float* cc1,
               const float* cc2) {
  const int half = dq / 2;
  const int F = heads * dq;
  dim3 grid(unsigned((ntok + TM - 1) / TM), unsigned(heads), 2u);
#define PKM_SCORE_CASE(NPLV)                                                                          \
  case NPLV: {                                                                                        \
    if constexpr ((TM / kWaves) * NPLV <= 64) { /* the plan never pairs a tall tile with wide rows */ \
      auto fn = score_topk_kernel<T, TM, NPLV>;                                                       \
      static LdsLimit lim; /* the largest plan's LDS, set once per device */                          \
      const hipError_t e = lim.ensure(reinterpret_cast<const void*>(fn), int(kLdsLimit));             \
      if (e != hipSuccess) return e;                                                                  \
      hipLaunchKernelGGL(fn, grid, dim3(kThreads), pl.lds, s, static_cast<const T*>(q), ntok, F, dq, half, \
                         pl.half_pad, pl.qstride, C, Cp, nk,                                           \
                         nk2, k, pl.cw, pl.sstride, sub_idx, sub_score, cc1, cc2);                   \
    }                                                                                                 \
  } break;
  switch (pl.npl) {
    PKM_SCORE_CASE(1)
    PKM_SCORE_CASE(2)
    PKM_SCORE_CASE(4)
    PKM_SCORE_CASE(8)
    PKM_SCORE_CASE(16)
    default:
      break;
  }
#undef PKM_SCORE_CASE
  return hipSuccess;
}

template <typename T>
hipError_t launch_t(hipStream_t s, const Plan& pl, const void* q, int64_t ntok, int heads, int dq, const u32x4* C,
              const u32x4* Cp, int nk, int nk2, int k, int32_t* sub_idx, float* sub_score, const float* cc1,
              const float* cc2) {
  if (pl.TM == 64) return launch_tm<T, 64>(s, pl, q, ntok, heads, dq, C, Cp, nk, nk2, k, sub_idx, sub_score, cc1, cc2);
  if (pl.TM == 32) return launch_tm<T, 32>(s, pl, q, ntok, heads, dq, C, Cp, nk, nk2, k, sub_idx, sub_score, cc1, cc2);
  return launch_tm<T, 16>(s, pl, q, ntok, heads, dq, C, Cp, nk, nk2, k, sub_idx, sub_score, cc1, cc2);
}

}  // namespace

bool score_topk_supported(int dtype, int half, int nkeys) {
  if (nkeys < 1 || nkeys > 2048) return false;
  Plan p = make_plan(dtype, half, nkeys);
  return p.TM != 0;
}

size_t score_topk_packed_bytes(int dtype, int heads, int half, int nk, int nk2) {
  const int KC = dtype == kBF16 ? 32 : 16;
  const size_t nks = size_t(round_up(half, KC) / KC);
  // packed operands, then the sub-key squared norms of the IDW scores
  const size_t own = size_t(heads) * (size_t((nk + 15) / 16) + size_t((nk2 + 15) / 16)) * nks * 64 * 16 +
                     size_t(heads) * size_t(nk + nk2) * 4;
  // the register-resident kernel's layout, where it may run instead
  const size_t sel = dtype == kBF16 ? score_select_packed_bytes(heads, half, nk, nk2) : 0;
  return own > sel ? own : sel;
}

hipError_t launch_score_topk(hipStream_t s, int dtype, const void* q, int64_t ntok, int heads, int dq,
                             const void* C, const void* Cp, int nk, int nk2, int k, int32_t* sub_idx,
                             float* sub_score, void* packed, bool idw, void* list) {
  const int half = dq / 2;
  if (score_select_supported(dtype, half, nk, nk2, k, idw))
    return launch_score_select(s, q, ntok, heads, dq, C, Cp, nk, nk2, k, sub_idx, sub_score, packed, list);
  int cus = 256;
  {
    int dev = 0;
    if (hipGetDevice(&dev) == hipSuccess) (void)hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev);
  }
  const bool few_tiles = (ntok + 31) / 32 * heads * 2 < cus;
  const Plan pl = make_plan(dtype, half, nk > nk2 ? nk : nk2, few_tiles);
  if (pl.TM == 0 || pl.npl > 16) return hipErrorInvalidValue;
  const int KC = dtype == kBF16 ? 32 : 16;
  const int nks = pl.half_pad / KC;
  u32x4* P1 = static_cast<u32x4*>(packed);
  u32x4* P2 = P1 + size_t(heads) * ((nk + 15) / 16) * nks * 64;
  const int64_t total = int64_t(heads) * ((nk + 15) / 16 + (nk2 + 15) / 16) * nks * 64;
  int64_t pb = (total + 255) / 256;
  if (pb > 4096) pb = 4096;
  float* cc1 = nullptr;
  float* cc2 = nullptr;
  int64_t nb = 0;
  if (idw) {  // |c|^2 after the packed operands: C's rows, then C''s
    cc1 = reinterpret_cast<float*>(P1 + total);
    cc2 = cc1 + size_t(heads) * nk;
    nb = (int64_t(heads) * (nk + nk2) + 3) / 4;  // four waves (rows) per block
    if (nb > 4096) nb = 4096;
  }
  if (dtype == kBF16)
    hipLaunchKernelGGL(pack_keys_kernel<bf16_t>, dim3(unsigned(pb + nb)), dim3(256), 0, s,
                       static_cast<const bf16_t*>(C), nk, static_cast<const bf16_t*>(Cp), nk2, heads, half, nks,
                       int(pb), P1, cc1);
  else
    hipLaunchKernelGGL(pack_keys_kernel<float>, dim3(unsigned(pb + nb)), dim3(256), 0, s,
                       static_cast<const float*>(C), nk, static_cast<const float*>(Cp), nk2, heads, half, nks,
                       int(pb), P1, cc1);
  const hipError_t e = dtype == kBF16
                           ? launch_t<bf16_t>(s, pl, q, ntok, heads, dq, P1, P2, nk, nk2, k, sub_idx, sub_score, cc1, cc2)
                           : launch_t<float>(s, pl, q, ntok, heads, dq, P1, P2, nk, nk2, k, sub_idx, sub_score, cc1, cc2);
  if (e != hipSuccess) return e;
  return hipGetLastError();
}

}  // namespace pkm
