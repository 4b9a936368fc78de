// Deterministic grouping for the sparse backward: a stable LSD radix sort of
// (key, lookup id) pairs, an exclusive scan, and the segment table of the
// sorted keys.  Only the selected rows / sub-keys receive gradient
// ("Meta AI 可扩展内存层", sections 6.1 and 9.2: sparse gradients at the
// selected positions; product-key paper summary: only a few memory slots are
// updated per step); grouping by a stable sort makes every per-row sum run in
// lookup order, so the backward is bit-identical from run to run without
// floating-point atomics.
//
// Radix pass (8-bit digit), two launches.  At most kSortBlocks blocks, block b
// owning the keys [b chunk, (b + 1) chunk) in sub-tiles of 1024 keys per wave.
// The first launch counts the digits of each block's chunk into a block-major
// (block, digit) table.  In the second each block first turns the table into
// its own write bases (the keys of smaller digits anywhere, plus the keys of
// its digit in earlier blocks: a few KB of table per block, read from L2), so
// no scan launch sits between the two.  Then, per sub-tile, each wave walks
// its 1024 keys 64 at a time, ranking every key among equal digits by matching
// the 8 digit bits with ballots and keeping per-digit counts in its own LDS
// row; one barrier turns the waves' counts into per-wave bases, and the keys,
// still in registers, are written out in index order per digit.
//
// Segments of a sorted key array are found in one scan over "key differs from
// its predecessor" computed on the fly: the apply pass (which sums the earlier
// blocks' counts itself) writes each segment's start (and key) at its rank
// directly.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int kScanBlock = 4096;
constexpr int kSortBlocks = 256;  // blocks of a radix pass at most (one per CU)

__device__ __forceinline__ int lanes_below(uint64_t m) {
  return __builtin_amdgcn_mbcnt_hi(uint32_t(m >> 32), __builtin_amdgcn_mbcnt_lo(uint32_t(m), 0u));
}

// Exclusive scan over the 256 threads of a block; returns the block total in *tot.
__device__ __forceinline__ uint32_t block_excl_scan(uint32_t v, uint32_t* sh /*[4]*/, uint32_t* tot) {
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
  uint32_t x = v;
#pragma unroll
  for (int d = 1; d < 64; d <<= 1) {
    uint32_t y = __shfl_up(x, d, 64);
    if (lane >= d) x += y;
  }
  if (lane == 63) sh[wave] = x;
  __syncthreads();
  uint32_t pre = 0, all = 0;
#pragma unroll
  for (int w = 0; w < 4; ++w) {
    if (w < wave) pre += sh[w];
    all += sh[w];
  }
  __syncthreads();
  *tot = all;
  return pre + x - v;
}

// Blocks of a radix pass: W waves (1024 W keys per sub-tile), nb blocks of
// chunk keys each (a multiple of the sub-tile).
struct RadixPlan {
  int waves, nb;
  int64_t chunk;
};

RadixPlan radix_plan(int64_t n) {
  RadixPlan p{};
  p.waves = n >= int64_t(kSortBlocks) * 8192 ? 16 : 4;  // 2 M keys and more: one 16-wave block per CU
  const int64_t sub = int64_t(1024) * p.waves;
  const int64_t subs = (n + sub - 1) / sub;
  const int64_t per = (subs + kSortBlocks - 1) / kSortBlocks;
  p.chunk = (per > 0 ? per : 1) * sub;
  p.nb = int((n + p.chunk - 1) / p.chunk);
  return p;
}

// Digit counts of one block's chunk.  Lanes holding the same digit are matched
// with ballots first, so each distinct digit of a wave takes one LDS atomic:
// skewed keys (a few hot rows or sub-keys) would otherwise serialise on one counter.
template <int W>
__global__ __launch_bounds__(64 * W) void radix_hist_kernel(const uint32_t* __restrict__ keys, int64_t n, int shift,
                                                            int64_t chunk, int nb, uint32_t* __restrict__ hist) {
  constexpr int NT = 64 * W;
  constexpr int G = W / 4;  // groups of four waves, each with its own counters
  __shared__ uint32_t cnts[G][256];
  for (int d = threadIdx.x; d < G * 256; d += NT) cnts[d >> 8][d & 255] = 0;
  __syncthreads();
  uint32_t* cnt = cnts[(threadIdx.x >> 6) / 4];
  const int64_t lo = int64_t(blockIdx.x) * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  for (int64_t base = lo; base < hi; base += 16 * NT) {
    uint32_t key[16];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const int64_t e = base + i * NT + threadIdx.x;
      key[i] = e < hi ? keys[e] : 0u;
    }
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      const bool ok = base + i * NT + threadIdx.x < hi;
      const uint32_t d = (key[i] >> shift) & 0xFF;
      uint64_t peers = ballot(ok);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
      }
      if (ok && lanes_below(peers) == 0) atomicAdd(&cnt[d], uint32_t(popc64(peers)));
    }
  }
  __syncthreads();
  if (threadIdx.x < 256) {
    uint32_t c = 0;
#pragma unroll
    for (int g = 0; g < G; ++g) c += cnts[g][threadIdx.x];
    hist[int64_t(blockIdx.x) * 256 + threadIdx.x] = c;
  }
}

// Stable scatter of one block's chunk.  vals_in == nullptr: the value is the key's index.
// Per sub-tile the ranked keys are first placed in LDS in digit order (each
// digit's keys in index order), then written out by consecutive threads: a
// digit's keys land in consecutive output positions, so the writes coalesce.
template <int W>
constexpr size_t radix_scatter_lds() {
  return size_t(1024) * W * 8 + size_t(W) * 256 * 4 + 2 * 256 * 4 + 16;
}

template <int W>
__global__ __launch_bounds__(64 * W) void radix_scatter_kernel(const uint32_t* __restrict__ keys_in,
                                                               const int32_t* __restrict__ vals_in, int64_t n,
                                                               int shift, int64_t chunk, int nb,
                                                               const uint32_t* __restrict__ hist,
                                                               uint32_t* __restrict__ keys_out,
                                                               int32_t* __restrict__ vals_out) {
  constexpr int NT = 64 * W;
  constexpr int SUB = 1024 * W;    // keys per sub-tile
  constexpr int PARTS = NT / 256;  // threads per digit summing the table
  constexpr int kRounds = 16;      // 64-key rounds per wave and sub-tile
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint32_t* lkey = reinterpret_cast<uint32_t*>(smem);                  // [SUB] sub-tile in digit order
  int32_t* lval = reinterpret_cast<int32_t*>(lkey + SUB);               // [SUB]
  uint32_t (*part)[PARTS][256] = reinterpret_cast<uint32_t (*)[PARTS][256]>(smem);  // prologue only (aliases lkey)
  uint32_t (*cnt)[256] = reinterpret_cast<uint32_t (*)[256]>(lval + SUB);  // [W][256] counts, then LDS bases
  uint32_t* run = &cnt[W][0];      // [256] output position of the digit's next key
  uint32_t* gbase = run + 256;     // [256] output position minus LDS position, this sub-tile
  uint32_t* wsum = gbase + 256;    // [4]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  {  // the digit's keys in earlier blocks (pre) and in all blocks (tot): thread (pp, d)
     // sums rows pp, pp + PARTS, ... of the block-major table, 16 rows in flight
    const int d = tid & 255, pp = tid >> 8;
    uint32_t pre = 0, tot = 0;
    for (int t0 = pp; t0 < nb; t0 += 16 * PARTS) {
      uint32_t v[16];
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        const int t = t0 + i * PARTS;
        v[i] = t < nb ? hist[int64_t(t) * 256 + d] : 0u;
      }
#pragma unroll
      for (int i = 0; i < 16; ++i) {
        tot += v[i];
        pre += t0 + i * PARTS < int(blockIdx.x) ? v[i] : 0u;
      }
    }
    part[0][pp][d] = pre;
    part[1][pp][d] = tot;
  }
  __syncthreads();
  {
    uint32_t pre = 0, tot = 0, x = 0;
    if (tid < 256) {
#pragma unroll
      for (int pp = 0; pp < PARTS; ++pp) {
        pre += part[0][pp][tid];
        tot += part[1][pp][tid];
      }
      x = tot;  // inclusive scan of the digit totals over the wave
#pragma unroll
      for (int dd = 1; dd < 64; dd <<= 1) {
        const uint32_t y = __shfl_up(x, dd, 64);
        if (lane >= dd) x += y;
      }
      if (lane == 63) wsum[wave] = x;
    }
    __syncthreads();
    if (tid < 256) {
      uint32_t below = 0;
      for (int w = 0; w < wave; ++w) below += wsum[w];
      run[tid] = below + x - tot + pre;
    }
  }
  const int64_t lo = int64_t(blockIdx.x) * chunk;
  const int64_t hi = lo + chunk < n ? lo + chunk : n;
  for (int64_t sb = lo; sb < hi; sb += SUB) {
    for (int d = lane; d < 256; d += 64) cnt[wave][d] = 0;
    const int64_t base = sb + int64_t(wave) * 1024;
    uint32_t key[kRounds];
    int32_t val[kRounds];
    uint32_t lpos[kRounds];
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int64_t e = base + i * 64 + lane;
      const bool ok = e < hi;
      key[i] = ok ? keys_in[e] : 0u;
      val[i] = ok ? (vals_in ? vals_in[e] : int32_t(e)) : 0;
    }
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      const int64_t e = base + i * 64 + lane;
      const bool ok = e < hi;
      const uint32_t d = (key[i] >> shift) & 0xFF;
      uint64_t peers = ballot(ok);
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const bool bit = (d >> b) & 1u;
        const uint64_t m = ballot(bit);
        peers &= bit ? m : ~m;
      }
      const int rk = lanes_below(peers);
      const uint32_t before = ok ? cnt[wave][d] : 0u;  // every lane reads before the leader writes
      lpos[i] = before + uint32_t(rk);
      if (ok && rk == 0) cnt[wave][d] = before + uint32_t(popc64(peers));
    }
    __syncthreads();  // counts done (and, on the first sub-tile, the prologue's reads of part)
    uint32_t tot = 0, x = 0;
    if (tid < 256) {  // the sub-tile's keys of digit tid, and their scan over the digits
#pragma unroll
      for (int w = 0; w < W; ++w) tot += cnt[w][tid];
      x = tot;
#pragma unroll
      for (int dd = 1; dd < 64; dd <<= 1) {
        const uint32_t y = __shfl_up(x, dd, 64);
        if (lane >= dd) x += y;
      }
      if (lane == 63) wsum[wave] = x;
    }
    __syncthreads();
    if (tid < 256) {  // LDS position of the digit's first key per wave; output offset
      uint32_t below = 0;
      for (int w = 0; w < wave; ++w) below += wsum[w];
      const uint32_t lst = below + x - tot;
      uint32_t r = lst;
#pragma unroll
      for (int w = 0; w < W; ++w) {
        const uint32_t c = cnt[w][tid];
        cnt[w][tid] = r;
        r += c;
      }
      gbase[tid] = run[tid] - lst;
      run[tid] += tot;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < kRounds; ++i) {
      if (base + i * 64 + lane < hi) {
        const uint32_t p = cnt[wave][(key[i] >> shift) & 0xFF] + lpos[i];
        lkey[p] = key[i];
        lval[p] = val[i];
      }
    }
    __syncthreads();
    const int ns = int(hi - sb < SUB ? hi - sb : SUB);
#pragma unroll 8
    for (int j = 0; j < SUB / NT; ++j) {
      const int i = j * NT + tid;
      if (i < ns) {
        const uint32_t kk = lkey[i];
        const uint32_t pos = gbase[(kk >> shift) & 0xFF] + uint32_t(i);
        keys_out[pos] = kk;
        vals_out[pos] = lval[i];
      }
    }
    __syncthreads();  // the next sub-tile reuses the LDS buffers and bases
  }
}

// Flag bits of the 16 sorted keys k[b0 .. b0+15] (bit i set when b0+i starts a
// segment: the first key or one that differs from its predecessor).  A full
// group is read with four 16-byte loads; the ragged tail element by element.
__device__ __forceinline__ uint32_t seg_flags16(const uint32_t* __restrict__ k, int64_t n, int64_t b0) {
  uint32_t v[16];
  if (b0 + 16 <= n && (reinterpret_cast<uintptr_t>(k) & 15u) == 0) {
    const uint4* p = reinterpret_cast<const uint4*>(k + b0);
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const uint4 q = p[j];
      v[4 * j] = q.x;
      v[4 * j + 1] = q.y;
      v[4 * j + 2] = q.z;
      v[4 * j + 3] = q.w;
    }
  } else {
#pragma unroll
    for (int i = 0; i < 16; ++i) v[i] = b0 + i < n ? k[b0 + i] : 0u;
  }
  uint32_t prev = b0 > 0 && b0 < n ? k[b0 - 1] : ~v[0];
  uint32_t f = 0;
#pragma unroll
  for (int i = 0; i < 16; ++i) {
    if (b0 + i < n && v[i] != prev) f |= 1u << i;
    prev = v[i];
  }
  return f;
}

// Segment scan over flag(i) = (i == 0 || k[i] != k[i-1]): per-block flag counts.
__global__ __launch_bounds__(256) void seg_reduce_kernel(const uint32_t* __restrict__ k, int64_t n,
                                                         uint32_t* __restrict__ part) {
  __shared__ uint32_t sh[4];
  const int64_t b0 = int64_t(blockIdx.x) * kScanBlock + threadIdx.x * 16;
  uint32_t tot;
  block_excl_scan(uint32_t(__popc(seg_flags16(k, n, b0))), sh, &tot);
  if (threadIdx.x == 0) part[blockIdx.x] = tot;
}

// Writes seg_start[rank] = i (and touched[rank] = k[i]) for every segment start
// i, the block's first rank being the sum of the earlier blocks' counts in part
// (nb entries, summed here); the last block also closes the table:
// seg_start[total] = n, *count = total.
__global__ __launch_bounds__(256) void seg_apply_kernel(const uint32_t* __restrict__ k, int64_t n,
                                                        const uint32_t* __restrict__ part, int nb,
                                                        int32_t* __restrict__ seg_start,
                                                        int32_t* __restrict__ touched, int64_t* __restrict__ count) {
  __shared__ uint32_t sh[4];
  uint32_t pre = 0, all = 0;
  for (int t = threadIdx.x; t < nb; t += 256) {
    const uint32_t v = part[t];
    all += v;
    pre += t < int(blockIdx.x) ? v : 0u;
  }
  uint32_t base, total;
  block_excl_scan(pre, sh, &base);
  block_excl_scan(all, sh, &total);
  const int64_t b0 = int64_t(blockIdx.x) * kScanBlock + threadIdx.x * 16;
  const uint32_t f = seg_flags16(k, n, b0);
  uint32_t tot;
  uint32_t rank = block_excl_scan(uint32_t(__popc(f)), sh, &tot) + base;
#pragma unroll
  for (int i = 0; i < 16; ++i)
    if (f & (1u << i)) {
      seg_start[rank] = int32_t(b0 + i);
      if (touched) touched[rank] = int32_t(k[b0 + i]);
      ++rank;
    }
  if (blockIdx.x == gridDim.x - 1 && threadIdx.x == 0) {
    seg_start[total] = int32_t(n);
    *count = int64_t(total);
  }
}

__global__ void seg_empty_kernel(int32_t* seg_start, int64_t* count) {
  if (threadIdx.x == 0) {
    seg_start[0] = 0;
    *count = 0;
  }
}

// ---------------------------------------------------------------------------
// Small batches (n <= kSmallSortMax): the whole grouping in one workgroup of
// 1024 threads, so a few thousand lookups cost one launch instead of a
// histogram, a scan and a scatter per digit plus the segment passes.  The
// (key, lookup id) pairs, packed as key << 32 | id, ping-pong between two LDS
// buffers.  Per digit (DB = 8 or 10 bits) each of the 16 waves owns a
// contiguous run of pairs, ranks them among equal digits with DB ballots and
// counts them in its own LDS row of 2^DB counters (as radix_scatter_kernel does
// per tile); one scan over (digit, wave)
// turns the counts into bases, and the pairs, still in registers, are written
// to the other buffer.  The order is stable, so equal keys keep their lookup
// order.  Then the segment table is built from the sorted keys in the same
// workgroup, and (plan_counts != null) the value gradient's long-run plan of
// those segments, from a copy of the segment starts in the free LDS buffer
// (LDS atomics hand out the chunk slots; the sums over a run's chunks are
// taken in chunk order, so the slot order does not matter).  10-bit digits
// sort 17- to 20-bit row ids in two passes instead of three; their 64 KB of
// counters fit beside the pairs up to kSmallWideMax pairs.
// ---------------------------------------------------------------------------
constexpr int kSmallThreads = 1024;
constexpr int kSmallWaves = kSmallThreads / 64;
constexpr int kSmallRounds = kSmallSortMax / kSmallWaves / 64;  // 64-pair rounds per wave at most
constexpr int kSmallPer = kSmallSortMax / kSmallThreads;        // keys per thread at most
constexpr int kSmallWideMax = 4096;  // pairs up to which 10-bit digits fit the LDS

// two pair buffers, a row of 2^DB digit counters per wave, 64 words of sums
size_t small_sort_lds_bytes(int64_t n, int db) {
  return size_t(n) * 16 + size_t(kSmallWaves) * (size_t(1) << db) * 4 + 64 * 4;
}

// Digit width of the one-workgroup sort: 10 bits where that saves a pass and
// the counters fit beside the pairs, else 8.
int small_digit_bits(int64_t n, int key_bits) {
  const int p8 = key_bits > 8 ? (key_bits + 7) / 8 : 1, p10 = key_bits > 10 ? (key_bits + 9) / 10 : 1;
  return n <= kSmallWideMax && p10 < p8 ? 10 : 8;
}

//
// Grouped (gridDim.x > 1): workgroup g sorts pairs [g n, (g + 1) n) on their
// own.  Its segment table (n + 1 entries, positions global) and touched keys
// go to group g's slice of seg_start / touched, its count to count[g].  Then
// either (plan_stride == 0) group_segments_kernel joins the tables into one
// (the caller guaranteeing that every key of group g is below every key of
// group g + 1, so the groups' sorted runs side by side are the sorted whole)
// and builds the long-run plan, or (plan_stride > 0) each group stays on its
// own and lists its own long runs in its own plan, plan_stride bytes after the
// previous group's (counts, chunk_list and long_list all move by it).
template <int DB>
__global__ __launch_bounds__(kSmallThreads) void small_sort_segments_kernel(
    const uint32_t* __restrict__ keys_in, int n, int passes, uint32_t* __restrict__ keys_out,
    int32_t* __restrict__ vals_out, int32_t* __restrict__ seg_start, int32_t* __restrict__ touched,
    int64_t* __restrict__ count, int chunk, int2* __restrict__ chunk_list, int2* __restrict__ long_list,
    uint32_t* __restrict__ plan_counts, int64_t plan_stride) {
  const int64_t base = int64_t(blockIdx.x) * n;  // this group's first pair
  if (gridDim.x > 1) {
    if (plan_stride == 0) {  // joined: the joining launch lists the long runs, into counters zeroed here
      if (blockIdx.x == 0 && threadIdx.x == 0 && plan_counts) plan_counts[0] = plan_counts[1] = 0u;
      plan_counts = nullptr;
    } else if (plan_counts) {  // separate groups: this group's own plan
      const int64_t off = int64_t(blockIdx.x) * plan_stride;
      plan_counts = reinterpret_cast<uint32_t*>(reinterpret_cast<char*>(plan_counts) + off);
      chunk_list = reinterpret_cast<int2*>(reinterpret_cast<char*>(chunk_list) + off);
      long_list = reinterpret_cast<int2*>(reinterpret_cast<char*>(long_list) + off);
    }
  }
  keys_in += base;
  keys_out += base;
  vals_out += base;
  seg_start += int64_t(blockIdx.x) * (n + 1);
  if (touched) touched += base;
  count += blockIdx.x;
  extern __shared__ __attribute__((aligned(16))) char smem[];
  uint64_t* bufA = reinterpret_cast<uint64_t*>(smem);
  uint64_t* bufB = bufA + n;
  constexpr int NB = 1 << DB;  // digits per pass
  uint32_t* cnt = reinterpret_cast<uint32_t*>(bufB + n);  // [kSmallWaves][NB]
  uint32_t* wsum = cnt + kSmallWaves * NB;                  // [64]
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  if (tid == 0) wsum[32] = wsum[33] = 0u;  // long-run plan counters
  {
    uint32_t kk[kSmallPer];  // every load in flight before the first store
#pragma unroll
    for (int r = 0; r < kSmallPer; ++r) {
      const int i = tid + r * kSmallThreads;
      kk[r] = i < n ? keys_in[i] : 0u;
    }
#pragma unroll
    for (int r = 0; r < kSmallPer; ++r) {
      const int i = tid + r * kSmallThreads;
      if (i < n) bufA[i] = (uint64_t(kk[r]) << 32) | uint32_t(base + i);
    }
  }
  // wave w owns pairs [w * per, (w + 1) * per), per a multiple of 64
  const int per = ((n + kSmallWaves - 1) / kSmallWaves + 63) / 64 * 64;
  const int rounds = per / 64;
  uint64_t* src = bufA;
  uint64_t* dst = bufB;
  for (int p = 0; p < passes; ++p) {
    const int shift = 32 + DB * p;
    for (int d = lane; d < NB; d += 64) cnt[wave * NB + d] = 0;
    __syncthreads();  // bufA filled / previous scatter done; counters cleared
    uint64_t kv[kSmallRounds];
    uint32_t lpos[kSmallRounds];
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
      if (r < rounds) {  // wave-uniform
        const int e = wave * per + r * 64 + lane;
        const bool ok = e < n;
        kv[r] = ok ? src[e] : 0ull;
        const uint32_t d = uint32_t(kv[r] >> shift) & uint32_t(NB - 1);
        uint64_t peers = ballot(ok);
#pragma unroll
        for (int b = 0; b < DB; ++b) {
          const bool bit = (d >> b) & 1u;
          const uint64_t m = ballot(bit);
          peers &= bit ? m : ~m;
        }
        const int rk = lanes_below(peers);
        const uint32_t before = ok ? cnt[wave * NB + d] : 0u;  // every lane reads before the leader writes
        lpos[r] = before + uint32_t(rk);
        if (ok && rk == 0) cnt[wave * NB + d] = before + uint32_t(popc64(peers));
      }
    }
    __syncthreads();
    // bases in (digit, wave) order: digit tid's total, scanned over the NB digits
    uint32_t tot = 0, incl = 0;
    if (tid < NB) {
      for (int w = 0; w < kSmallWaves; ++w) tot += cnt[w * NB + tid];
      incl = tot;
#pragma unroll
      for (int dd = 1; dd < 64; dd <<= 1) {
        const uint32_t y = __shfl_up(incl, dd, 64);
        if (lane >= dd) incl += y;
      }
      if (lane == 63) wsum[wave] = incl;
    }
    __syncthreads();
    if (tid < NB) {
      uint32_t run = incl - tot;
      for (int w = 0; w < wave; ++w) run += wsum[w];
      for (int w = 0; w < kSmallWaves; ++w) {
        const uint32_t c = cnt[w * NB + tid];
        cnt[w * NB + tid] = run;
        run += c;
      }
    }
    __syncthreads();
#pragma unroll
    for (int r = 0; r < kSmallRounds; ++r) {
      if (r < rounds) {
        const int e = wave * per + r * 64 + lane;
        if (e < n) {
          const uint32_t d = uint32_t(kv[r] >> shift) & uint32_t(NB - 1);
          dst[cnt[wave * NB + d] + lpos[r]] = kv[r];
        }
      }
    }
    uint64_t* t = src;
    src = dst;
    dst = t;
  }
  __syncthreads();
  // sorted pairs out; segment starts: the first key and every key that differs from its predecessor
  for (int i = tid; i < n; i += kSmallThreads) {
    keys_out[i] = uint32_t(src[i] >> 32);
    vals_out[i] = int32_t(uint32_t(src[i]));  // the pair's global index
  }
  const int ipt = (n + kSmallThreads - 1) / kSmallThreads;
  const int i0 = tid * ipt;
  uint32_t flags = 0;
  for (int j = 0; j < ipt; ++j) {
    const int i = i0 + j;
    if (i < n && (i == 0 || uint32_t(src[i] >> 32) != uint32_t(src[i - 1] >> 32))) flags |= 1u << j;
  }
  const uint32_t c = uint32_t(__popc(flags));
  uint32_t x = c;
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const uint32_t y = __shfl_up(x, dd, 64);
    if (lane >= dd) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t rank = x - c, total = 0;
  for (int w = 0; w < kSmallWaves; ++w) {
    if (w < wave) rank += wsum[w];
    total += wsum[w];
  }
  int32_t* segl = reinterpret_cast<int32_t*>(dst);  // free after the passes: room for 2n ints
  const bool plan = plan_counts != nullptr && n > 0;
  for (int j = 0; j < ipt; ++j) {
    if (flags & (1u << j)) {
      seg_start[rank] = int32_t(base + i0 + j);
      if (touched) touched[rank] = int32_t(src[i0 + j] >> 32);
      if (plan) segl[rank] = i0 + j;
      ++rank;
    }
  }
  if (tid == 0) {
    seg_start[total] = int32_t(base + n);
    *count = int64_t(total);
    if (plan) segl[total] = n;
  }
  if (plan_counts == nullptr) return;  // uniform over the workgroup
  __syncthreads();
  for (int u = tid; u < int(total); u += kSmallThreads) {
    const int lo = segl[u];
    const int len = segl[u + 1] - lo;
    if (len > chunk) {
      const int nch = (len + chunk - 1) / chunk;
      const uint32_t base = atomicAdd(&wsum[32], uint32_t(nch));
      for (int j = 0; j < nch; ++j) chunk_list[base + j] = make_int2(u, j);
      long_list[atomicAdd(&wsum[33], 1u)] = make_int2(u, int(base));
    }
  }
  __syncthreads();
  if (tid == 0) {
    plan_counts[0] = wsum[32];
    plan_counts[1] = wsum[33];
  }
}

// Joins the groups' segment tables (seg_g: group g's n_per + 1 entries at
// g (n_per + 1), the last one its end; touched_g at g n_per; cnt_g[g]
// segments) into one table of all n = groups * n_per pairs, and lists the
// value gradient's long runs as long_run_plan_kernel does (plan counts zeroed
// before, by the sorting launch).  Every block scans the group counts itself
// (groups <= kSortGroupsMax) and takes a grid-stride share of the segments; a
// run's length comes from its own group's table, so no block reads what
// another writes.
constexpr int kJoinThreads = 256;
__global__ __launch_bounds__(kJoinThreads) void group_segments_kernel(
    const int32_t* __restrict__ seg_g, const int32_t* __restrict__ touched_g, const int64_t* __restrict__ cnt_g,
    int groups, int n_per, int32_t* __restrict__ seg_start, int32_t* __restrict__ touched,
    int64_t* __restrict__ count, int chunk, int2* __restrict__ chunk_list, int2* __restrict__ long_list,
    uint32_t* __restrict__ plan_counts, int64_t end_pos) {
  constexpr int kPer = kSortGroupsMax / kJoinThreads;  // group counts per thread
  __shared__ uint32_t offs[kSortGroupsMax + 1];
  __shared__ uint32_t wsum[kJoinThreads / 64];
  const int tid = threadIdx.x, lane = tid & 63, wave = tid >> 6;
  uint32_t c[kPer], my = 0;
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    const int g = tid * kPer + q;
    c[q] = g < groups ? uint32_t(cnt_g[g]) : 0u;
    my += c[q];
  }
  uint32_t x = my;
#pragma unroll
  for (int dd = 1; dd < 64; dd <<= 1) {
    const uint32_t y = __shfl_up(x, dd, 64);
    if (lane >= dd) x += y;
  }
  if (lane == 63) wsum[wave] = x;
  __syncthreads();
  uint32_t pre = x - my, total = 0;
  for (int w = 0; w < kJoinThreads / 64; ++w) {
    if (w < wave) pre += wsum[w];
    total += wsum[w];
  }
#pragma unroll
  for (int q = 0; q < kPer; ++q) {
    offs[tid * kPer + q] = pre;
    pre += c[q];
  }
  if (tid == 0) offs[kSortGroupsMax] = total;
  __syncthreads();
  const uint32_t stride = gridDim.x * kJoinThreads;
  for (uint32_t u = blockIdx.x * kJoinThreads + tid; u < total; u += stride) {
    int lo = 0, hi = groups - 1;  // the group holding segment u: the last g with offs[g] <= u
    while (lo < hi) {
      const int mid = (lo + hi + 1) / 2;
      if (offs[mid] <= u) lo = mid; else hi = mid - 1;
    }
    const uint32_t j = u - offs[lo];
    const int32_t* sg = seg_g + int64_t(lo) * (n_per + 1);
    const int32_t a = sg[j], len = sg[j + 1] - a;
    seg_start[u] = a;
    if (touched) touched[u] = touched_g[int64_t(lo) * n_per + j];
    if (len > chunk) {
      const int nch = (len + chunk - 1) / chunk;
      const uint32_t b = atomicAdd(&plan_counts[0], uint32_t(nch));
      for (int q = 0; q < nch; ++q) chunk_list[b + q] = make_int2(int(u), q);
      long_list[atomicAdd(&plan_counts[1], 1u)] = make_int2(int(u), int(b));
    }
  }
  if (blockIdx.x == 0 && tid == 0) {
    seg_start[total] = int32_t(end_pos);  // the position after the groups' last pair
    *count = int64_t(total);
  }
}

__global__ void zero_plan_counts_kernel(uint32_t* counts) {
  if (threadIdx.x < 2) counts[threadIdx.x] = 0u;
}

// The one-workgroup sort's LDS limits, raised to what each digit width's
// largest batch needs.
hipError_t small_sort_lds_limit() {
  static LdsLimit lim8, lim10;
  const hipError_t e = lim8.ensure(reinterpret_cast<const void*>(small_sort_segments_kernel<8>),
                                   int(small_sort_lds_bytes(kSmallSortMax, 8)));
  if (e != hipSuccess) return e;
  return lim10.ensure(reinterpret_cast<const void*>(small_sort_segments_kernel<10>),
                      int(small_sort_lds_bytes(kSmallWideMax, 10)));
}

// The one-workgroup sort with digits of db (8 or 10) bits.
void launch_small_sort(int db, dim3 grid, size_t lds, hipStream_t s, const uint32_t* keys_in, int n, int passes,
                       uint32_t* keys_out, int32_t* vals_out, int32_t* seg_start, int32_t* touched, int64_t* count,
                       int chunk, int2* chunk_list, int2* long_list, uint32_t* plan_counts, int64_t plan_stride) {
  if (db == 10)
    hipLaunchKernelGGL(small_sort_segments_kernel<10>, grid, dim3(kSmallThreads), lds, s, keys_in, n, passes, keys_out,
                       vals_out, seg_start, touched, count, chunk, chunk_list, long_list, plan_counts, plan_stride);
  else
    hipLaunchKernelGGL(small_sort_segments_kernel<8>, grid, dim3(kSmallThreads), lds, s, keys_in, n, passes, keys_out,
                       vals_out, seg_start, touched, count, chunk, chunk_list, long_list, plan_counts, plan_stride);
}

// Digits of db bits for keys of key_bits bits: the passes (at least one).
int small_passes(int key_bits, int db) {
  const int p = (key_bits + db - 1) / db;
  return p < 1 ? 1 : p > 4 ? 4 : p;
}

inline unsigned grid1d(int64_t n, int64_t cap = 16384) {
  int64_t b = (n + 255) / 256;
  if (b > cap) b = cap;
  if (b < 1) b = 1;
  return unsigned(b);
}

template <int W>
hipError_t radix_pass(hipStream_t s, const uint32_t* kin, const int32_t* vin, int64_t n, int shift,
                      const RadixPlan& pl, uint32_t* hist, uint32_t* kout, int32_t* vout) {
  static LdsLimit lim;  // dynamic LDS above 64 KB, raised once per device
  constexpr size_t lds = radix_scatter_lds<W>();
  const hipError_t e = lim.ensure(reinterpret_cast<const void*>(radix_scatter_kernel<W>), int(lds));
  if (e != hipSuccess) return e;
  hipLaunchKernelGGL(radix_hist_kernel<W>, dim3(unsigned(pl.nb)), dim3(64 * W), 0, s, kin, n, shift, pl.chunk, pl.nb,
                     hist);
  hipLaunchKernelGGL(radix_scatter_kernel<W>, dim3(unsigned(pl.nb)), dim3(64 * W), lds, s, kin, vin, n, shift,
                     pl.chunk, pl.nb, hist, kout, vout);
  return hipSuccess;
}

}  // namespace

size_t scan_temp_bytes(int64_t n) {
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  return size_t((nb + 64) * 4);
}

size_t radix_sort_temp_bytes(int64_t n) { return size_t(256) * radix_plan(n).nb * 4 + 256; }

hipError_t launch_radix_sort_from(hipStream_t s, const uint32_t* keys_in, uint32_t* k0, int32_t* v0, uint32_t* k1,
                                  int32_t* v1, int64_t n, int key_bits, void* temp, bool* result_in_1) {
  const RadixPlan pl = radix_plan(n);
  uint32_t* hist = static_cast<uint32_t*>(temp);
  int passes = (key_bits + 7) / 8;
  if (passes < 1) passes = 1;
  const uint32_t* kin = keys_in;
  const int32_t* vin = nullptr;
  uint32_t* kout = k0;
  int32_t* vout = v0;
  for (int p = 0; p < passes; ++p) {
    const int shift = 8 * p;
    if (pl.nb > 0) {
      hipError_t e = hipSuccess;
      if (pl.waves == 16)
        e = radix_pass<16>(s, kin, vin, n, shift, pl, hist, kout, vout);
      else if (pl.waves == 8)
        e = radix_pass<8>(s, kin, vin, n, shift, pl, hist, kout, vout);
      else
        e = radix_pass<4>(s, kin, vin, n, shift, pl, hist, kout, vout);
      if (e != hipSuccess) return e;
    }
    kin = kout;
    vin = vout;
    if (kout == k0) {
      kout = k1;
      vout = v1;
    } else {
      kout = k0;
      vout = v0;
    }
  }
  *result_in_1 = (kin == k1);
  return hipGetLastError();
}

size_t sort_groups_temp_bytes(int64_t n) {
  return size_t(n + kSortGroupsMax) * 4 + size_t(n) * 4 + size_t(kSortGroupsMax) * 8 + 64;
}

hipError_t launch_sort_segments_grouped(hipStream_t s, const uint32_t* keys_in, int64_t n, int groups,
                                        int key_bits, uint32_t* keys_out, int32_t* vals_out, int32_t* seg_start,
                                        int32_t* touched, int64_t* count, const VgPlan* plan, void* temp) {
  if (groups < 1 || groups > kSortGroupsMax || n % groups || n / groups > kSmallSortMax || plan == nullptr)
    return hipErrorInvalidValue;
  const int n_per = int(n / groups);
  {
    const hipError_t e = small_sort_lds_limit();
    if (e != hipSuccess) return e;
  }
  const int db = small_digit_bits(n_per, key_bits);
  const int passes = small_passes(key_bits, db);
  int32_t* seg_g = static_cast<int32_t*>(temp);             // groups x (n_per + 1)
  int32_t* touched_g = seg_g + n + kSortGroupsMax;          // groups x n_per
  int64_t* cnt_g = reinterpret_cast<int64_t*>(touched_g + n);  // groups (8-byte aligned: n + n + 1024 ints)
  launch_small_sort(db, dim3(unsigned(groups)), small_sort_lds_bytes(n_per, db), s, keys_in, n_per, passes, keys_out,
                    vals_out, seg_g, touched_g, cnt_g, kVgChunk, static_cast<int2*>(nullptr),
                    static_cast<int2*>(nullptr), plan->counts, int64_t(0));
  int64_t jb = (n + kJoinThreads - 1) / kJoinThreads;
  if (jb > 1024) jb = 1024;
  hipLaunchKernelGGL(group_segments_kernel, dim3(unsigned(jb)), dim3(kJoinThreads), 0, s, seg_g, touched_g, cnt_g,
                     groups, n_per, seg_start, touched, count, kVgChunk, plan->chunk_list, plan->long_list,
                     plan->counts, int64_t(groups) * n_per);
  return hipGetLastError();
}

hipError_t launch_sort_segments_small(hipStream_t s, const uint32_t* keys_in, int64_t n, int key_bits,
                                      uint32_t* keys_out, int32_t* vals_out, int32_t* seg_start, int32_t* touched,
                                      int64_t* count, const VgPlan* plan) {
  if (n < 0 || n > kSmallSortMax) return hipErrorInvalidValue;
  {
    const hipError_t e = small_sort_lds_limit();
    if (e != hipSuccess) return e;
  }
  const int db = small_digit_bits(n, key_bits);
  const int passes = small_passes(key_bits, db);
  launch_small_sort(db, dim3(1), small_sort_lds_bytes(n, db), s, keys_in, int(n), passes, keys_out, vals_out,
                    seg_start, touched, count, kVgChunk, plan ? plan->chunk_list : static_cast<int2*>(nullptr),
                    plan ? plan->long_list : static_cast<int2*>(nullptr),
                    plan ? plan->counts : static_cast<uint32_t*>(nullptr), int64_t(0));
  return hipGetLastError();
}

size_t group_plan_stride() {
  const size_t slots = 2 * (kSmallSortMax / kVgChunk) + 2;
  return (64 + 2 * slots * sizeof(int2) + 255) / 256 * 256;
}

VgPlan group_plan(void* plans, int g) {
  const size_t slots = 2 * (kSmallSortMax / kVgChunk) + 2;
  char* b = static_cast<char*>(plans) + size_t(g) * group_plan_stride();
  VgPlan p;
  p.counts = reinterpret_cast<uint32_t*>(b);
  p.chunk_list = reinterpret_cast<int2*>(b + 64);
  p.long_list = p.chunk_list + slots;
  return p;
}

hipError_t launch_join_groups(hipStream_t s, const int32_t* seg_g, const int64_t* cnt_g, int groups, int n_per,
                              int64_t end_pos, int32_t* seg_start, int64_t* count, const VgPlan* plan) {
  if (groups < 1 || groups > kSortGroupsMax || n_per < 0 || plan == nullptr) return hipErrorInvalidValue;
  hipLaunchKernelGGL(zero_plan_counts_kernel, dim3(1), dim3(64), 0, s, plan->counts);
  int64_t jb = (int64_t(groups) * n_per + kJoinThreads - 1) / kJoinThreads;
  if (jb > 1024) jb = 1024;
  if (jb < 1) jb = 1;
  hipLaunchKernelGGL(group_segments_kernel, dim3(unsigned(jb)), dim3(kJoinThreads), 0, s, seg_g,
                     static_cast<const int32_t*>(nullptr), cnt_g, groups, n_per, seg_start,
                     static_cast<int32_t*>(nullptr), count, kVgChunk, plan->chunk_list, plan->long_list, plan->counts,
                     end_pos);
  return hipGetLastError();
}

hipError_t launch_sort_segments_separate(hipStream_t s, const uint32_t* keys_in, int64_t n, int groups, int key_bits,
                                         uint32_t* keys_out, int32_t* vals_out, int32_t* seg_g, int64_t* cnt_g,
                                         void* plans) {
  if (groups < 1 || groups > kSortGroupsMax || n % groups || n / groups > kSmallSortMax || plans == nullptr)
    return hipErrorInvalidValue;
  const int n_per = int(n / groups);
  {
    const hipError_t e = small_sort_lds_limit();
    if (e != hipSuccess) return e;
  }
  const int db = small_digit_bits(n_per, key_bits);
  const int passes = small_passes(key_bits, db);
  const VgPlan p0 = group_plan(plans, 0);
  launch_small_sort(db, dim3(unsigned(groups)), small_sort_lds_bytes(n_per, db), s, keys_in, n_per, passes, keys_out,
                    vals_out, seg_g, static_cast<int32_t*>(nullptr), cnt_g, kVgChunk, p0.chunk_list, p0.long_list,
                    p0.counts, int64_t(group_plan_stride()));
  return hipGetLastError();
}

hipError_t launch_segments(hipStream_t s, const uint32_t* sorted_keys, int64_t n, int32_t* seg_start,
                           int32_t* touched, int64_t* count, void* scan_temp) {
  uint32_t* part = static_cast<uint32_t*>(scan_temp);
  const int64_t nb = (n + kScanBlock - 1) / kScanBlock;
  if (nb > (int64_t(1) << 20)) return hipErrorInvalidValue;
  if (nb > 0) {
    hipLaunchKernelGGL(seg_reduce_kernel, dim3(unsigned(nb)), dim3(256), 0, s, sorted_keys, n, part);
    hipLaunchKernelGGL(seg_apply_kernel, dim3(unsigned(nb)), dim3(256), 0, s, sorted_keys, n, part, int(nb),
                       seg_start, touched, count);
  } else {
    hipLaunchKernelGGL(seg_empty_kernel, dim3(1), dim3(64), 0, s, seg_start, count);
  }
  return hipGetLastError();
}

}  // namespace pkm
