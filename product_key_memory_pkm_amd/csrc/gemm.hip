// Dense matrix products of the query network (steps a1 and a10):
//   forward  q_pre = x W_q^T                 (M = T,    N = h*dq, K = d)
//   backward dW_q  = dq_pre^T x              (M = h*dq, N = d,    K = T, split over K)
//            dx    = dq_pre W_q              (M = T,    N = d,    K = h*dq)
// all as C[M, N] = A[M, K] B[N, K]^T with both operands K-contiguous.
// ("Meta AI 可扩展内存层", sections 3.2 and 10.1: bias-free linear query
// projection; product-key paper summary, method details: every parameter is
// trained by back-propagation.)
//
// bf16 (K a multiple of 32, operands under 4 GB): 256x256 output tile per
// 8-wave workgroup (4 x 2 waves of 64 x 128), v_mfma_f32_32x32x16_bf16 with
// fp32 accumulation (gfx950 sustains about twice the bf16 flops with the
// 32x32x16 shape as with 16x16x32, for the same operand bytes read from LDS).  Operands go straight from memory into LDS with
// buffer_load ... lds (no register staging), five 32-deep K stages of 32 KB
// (the whole 160 KB of LDS) so that four are in flight while one is consumed;
// rows past the matrix read as zero through the buffer range check.  Each
// 16-row x 64-byte LDS block keeps its 16-byte chunks XOR-swizzled by row so
// the MFMA fragment reads of 16 rows spread over all banks.  Tiles are
// assigned so that each XCD (workgroups b with equal b % 8) walks a
// contiguous range of output rows, sharing the A panel in its L2.
//
// Otherwise: 128x128 output tile per 256-thread workgroup, 2x2 waves of
// 64x64, K staged through double-buffered LDS in 128-byte slices (64 bf16 or
// 32 fp32; fp32 uses v_mfma_f32_16x16x4f32); the next slice is fetched into
// registers while the current one feeds the MFMAs; rows padded by 16 bytes.
#include "common.h"
#include "kernels.h"

namespace pkm {

namespace {

constexpr int BM = 128, BN = 128;
constexpr int ROWB = 128;           // bytes of K per LDS row and stage
constexpr int LDSROW = ROWB + 16;   // padded row pitch (bytes)

template <typename T>
struct GemmTraits;
template <>
struct GemmTraits<bf16_t> {
  static constexpr int VE = 8;
  __device__ __forceinline__ static f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(bf16x8, a),
                                                    __builtin_bit_cast(bf16x8, b), c, 0, 0, 0);
  }
};
template <>
struct GemmTraits<float> {
  static constexpr int VE = 4;
  __device__ __forceinline__ static f32x4 mma(const u32x4& a, const u32x4& b, f32x4 c) {
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.x), __uint_as_float(b.x), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.y), __uint_as_float(b.y), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.z), __uint_as_float(b.z), c, 0, 0, 0);
    c = __builtin_amdgcn_mfma_f32_16x16x4f32(__uint_as_float(a.w), __uint_as_float(b.w), c, 0, 0, 0);
    return c;
  }
};

template <typename T>
__global__ __launch_bounds__(256) void gemm_nt_kernel(int64_t M, int64_t N, int64_t K, const T* __restrict__ A,
                                                      int64_t lda, const T* __restrict__ B, int64_t ldb,
                                                      void* __restrict__ Cout, int64_t ldc, int out_bf16,
                                                      int64_t kchunk, int64_t split_stride) {
  using TR = GemmTraits<T>;
  constexpr int VE = TR::VE;          // elements per 16-byte vector
  constexpr int BK = ROWB / sizeof(T);  // elements of K per stage
  __shared__ __attribute__((aligned(16))) char As[2][BM * LDSROW];
  __shared__ __attribute__((aligned(16))) char Bs[2][BN * LDSROW];

  const int tid = threadIdx.x;
  const int wave = tid >> 6, lane = tid & 63;
  const int wm = wave >> 1, wn = wave & 1;
  const int64_t m0 = int64_t(blockIdx.y) * BM;
  const int64_t n0 = int64_t(blockIdx.x) * BN;
  const int64_t kbeg = int64_t(blockIdx.z) * kchunk;
  const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;

  // global -> register loader: 1024 16-byte chunks per operand tile, 4 per thread
  u32x4 ra[4], rb[4];
  auto gload = [&](int64_t k0) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i;
      const int r = ch >> 3, kc = (ch & 7) * VE;
      const int64_t kk = k0 + kc;
      const int64_t am = m0 + r, bn = n0 + r;
      ra[i] = (am < M && kk < kend) ? ld16(A + am * lda + kk) : u32x4{0, 0, 0, 0};
      rb[i] = (bn < N && kk < kend) ? ld16(B + bn * ldb + kk) : u32x4{0, 0, 0, 0};
    }
  };
  auto sstore = [&](int buf) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int ch = tid + 256 * i;
      const int r = ch >> 3, kb = (ch & 7) * 16;
      st16(As[buf] + r * LDSROW + kb, ra[i]);
      st16(Bs[buf] + r * LDSROW + kb, rb[i]);
    }
  };

  f32x4 acc[4][4];
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

  const int lrow = lane & 15, lgrp = lane >> 4;
  const int nkt = kend > kbeg ? int((kend - kbeg + BK - 1) / BK) : 0;
  if (nkt > 0) {
    gload(kbeg);
    sstore(0);
  }
  __syncthreads();
  for (int kt = 0; kt < nkt; ++kt) {
    const int buf = kt & 1;
    if (kt + 1 < nkt) gload(kbeg + int64_t(kt + 1) * BK);
#pragma unroll
    for (int ks = 0; ks < 2; ++ks) {  // two 64-byte K sub-slices per stage
      u32x4 a[4], b[4];
      const int kb = ks * 64 + lgrp * 16;
#pragma unroll
      for (int i = 0; i < 4; ++i) a[i] = ld16(As[buf] + (wm * 64 + i * 16 + lrow) * LDSROW + kb);
#pragma unroll
      for (int j = 0; j < 4; ++j) b[j] = ld16(Bs[buf] + (wn * 64 + j * 16 + lrow) * LDSROW + kb);
#pragma unroll
      for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int j = 0; j < 4; ++j) acc[i][j] = TR::mma(a[i], b[j], acc[i][j]);
    }
    if (kt + 1 < nkt) sstore(buf ^ 1);
    __syncthreads();
  }

  // epilogue: lane holds column lrow and rows 4*lgrp + r of each 16x16 tile
  char* Cb = reinterpret_cast<char*>(Cout) + int64_t(blockIdx.z) * split_stride * (out_bf16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < 4; ++i)
#pragma unroll
    for (int j = 0; j < 4; ++j) {
      const int64_t col = n0 + wn * 64 + j * 16 + lrow;
      if (col >= N) continue;
#pragma unroll
      for (int r = 0; r < 4; ++r) {
        const int64_t row = m0 + wm * 64 + i * 16 + lgrp * 4 + r;
        if (row < M) {
          if (out_bf16)
            reinterpret_cast<uint16_t*>(Cb)[row * ldc + col] = f32_to_bf16(acc[i][j][r]);
          else
            reinterpret_cast<float*>(Cb)[row * ldc + col] = acc[i][j][r];
        }
      }
    }
}


// ---------------------------------------------------------------------------
// bf16 path with LDS-DMA operand staging
// ---------------------------------------------------------------------------
typedef __attribute__((ext_vector_type(4))) int i32x4;

// Buffer resource of `bytes` bytes at base (raw buffer: stride 0; reads at or
// beyond `bytes` return zero).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
  const uint64_t a = reinterpret_cast<uint64_t>(base);
  return i32x4{int(uint32_t(a)), int(uint32_t(a >> 32) & 0xFFFF), int(bytes), 0x00020000};
}
__device__ __forceinline__ uint32_t lds_addr(const char* p) {
  return uint32_t(reinterpret_cast<uintptr_t>((const __attribute__((address_space(3))) char*)(p)));
}
// 16 bytes per lane from buffer offset voff into LDS at lds_base + lane * 16.
// Written as asm because the compiler, seeing the builtin's LDS write, waits for
// every outstanding load before any later LDS read, which would drain the
// pipeline each K stage; the caller waits with s_waitcnt vmcnt instead.  The
// instruction has no register results (the data lands in LDS), and its address
// operands are read at issue.
__device__ __forceinline__ void dma16(i32x4 rsrc, uint32_t voff, uint32_t lds_base) {
  asm volatile("s_mov_b32 m0, %2\n\tbuffer_load_dwordx4 %0, %1, 0 offen lds"
               :
               : "v"(voff), "s"(rsrc), "s"(__builtin_amdgcn_readfirstlane(lds_base))
               : "memory", "m0");
}
// Workgroup barrier that orders LDS only (leaves later stages' loads in flight).
__device__ __forceinline__ void lds_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}
// s_waitcnt vmcnt(n) (n < 64), other counters untouched
#define PKM_WAIT_VM(n) __builtin_amdgcn_s_waitcnt(0x0F70 | ((n) & 0xF) | (((n) >> 4) << 14))

constexpr int kDmaStages = 5;
constexpr int kDmaStage = 32768;  // bytes per stage: A and B blocks of 256 rows x 64 bytes
constexpr int kDmaWM = 4, kDmaWN = 2;

__global__ __launch_bounds__(512) void gemm_nt_dma_kernel(int64_t M, int64_t N, const bf16_t* __restrict__ A,
                                                          int64_t lda, const bf16_t* __restrict__ B, int64_t ldb,
                                                          void* __restrict__ Cout, int64_t ldc, int out_bf16,
                                                          int64_t K, int64_t kchunk, int64_t split_stride,
                                                          double* __restrict__ bn_part) {
  constexpr int BM = 256, BN = 256, NW = kDmaWM * kDmaWN, TI = BM / kDmaWM / 32, TJ = BN / kDmaWN / 32;
  constexpr int BPW = 16 / NW;        // 1 KB blocks per operand, stage and wave
  constexpr int PER = 2 * BPW;        // DMA instructions per stage and wave
  extern __shared__ __attribute__((aligned(1024))) char smem[];
  const int tid = threadIdx.x, wave = tid >> 6, lane = tid & 63;
  const int wm = wave / kDmaWN, wn = wave % kDmaWN;
  const int64_t gx = (N + BN - 1) / BN, total = gx * ((M + BM - 1) / BM);
  int64_t t = blockIdx.x;
  if (total % 8 == 0) t = (t % 8) * (total / 8) + t / 8;  // XCD b % 8 gets a contiguous run of tiles
  const int64_t m0 = (t / gx) * BM, n0 = (t % gx) * BN;
  const int64_t kbeg = int64_t(blockIdx.y) * kchunk;
  const int64_t kend = kbeg + kchunk < K ? kbeg + kchunk : K;
  const i32x4 ra = make_rsrc(A, uint32_t(M * lda * 2));
  const i32x4 rb = make_rsrc(B, uint32_t(N * ldb * 2));
  // lane slot in a 1 KB block (16 rows x 64 bytes): row r, chunk position lane & 3, source chunk c
  const int r = lane >> 2, c = (lane & 3) ^ ((r >> 2) & 3);
  constexpr uint32_t kOut = 0xFFFFFFF0u;  // offset past any buffer: reads zero
  uint32_t aoff[BPW], boff[BPW];
#pragma unroll
  for (int i = 0; i < BPW; ++i) {
    const int64_t ar = m0 + (wave + NW * i) * 16 + r, br = n0 + (wave + NW * i) * 16 + r;
    aoff[i] = ar < M ? uint32_t((ar * lda + kbeg + c * 8) * 2) : kOut;
    boff[i] = br < N ? uint32_t((br * ldb + kbeg + c * 8) * 2) : kOut;
  }
  const int nkt = kend > kbeg ? int((kend - kbeg) / 32) : 0;
  auto issue = [&](int kt) {
    char* st = smem + (kt % kDmaStages) * kDmaStage;
    const uint32_t kb = uint32_t(kt) * 64;
#pragma unroll
    for (int i = 0; i < BPW; ++i) {
      dma16(ra, aoff[i] == kOut ? kOut : aoff[i] + kb, lds_addr(st + (wave + NW * i) * 1024));
      dma16(rb, boff[i] == kOut ? kOut : boff[i] + kb, lds_addr(st + 16384 + (wave + NW * i) * 1024));
    }
  };
  f32x16 acc[TI][TJ];
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j)
#pragma unroll
      for (int e = 0; e < 16; ++e) acc[i][j][e] = 0.f;
  // 32x32x16 operand fragments: lane l holds row (or column) l % 32 of a 32-row
  // tile (two 1 KB blocks) and k = 8 (l / 32) .. +8 of the 16-deep half h of the
  // stage, i.e. 16-byte chunk 2h + l / 32 of that row (swizzled as stored)
  const int fr_r = lane & 15, fr_hi = lane >> 5;
  const int fr_base = ((lane >> 4) & 1) * 1024 + fr_r * 64;
  const int fr0 = fr_base + (((0 + fr_hi) ^ ((fr_r >> 2) & 3)) * 16);
  const int fr1 = fr_base + (((2 + fr_hi) ^ ((fr_r >> 2) & 3)) * 16);
#pragma unroll
  for (int st = 0; st < kDmaStages - 1; ++st)
    if (st < nkt) issue(st);
  for (int kt = 0; kt < nkt; ++kt) {
    if (kt + kDmaStages - 1 < nkt) {
      issue(kt + kDmaStages - 1);
      PKM_WAIT_VM(PER * (kDmaStages - 1));  // stage kt landed; the next four stay in flight
    } else {
      PKM_WAIT_VM(0);
    }
    lds_barrier();
    const char* st = smem + (kt % kDmaStages) * kDmaStage;
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int fr = h ? fr1 : fr0;
      u32x4 b[TJ], a[TI];
#pragma unroll
      for (int j = 0; j < TJ; ++j) b[j] = *reinterpret_cast<const u32x4*>(st + 16384 + (wn * TJ + j) * 2048 + fr);
#pragma unroll
      for (int i = 0; i < TI; ++i) a[i] = *reinterpret_cast<const u32x4*>(st + (wm * TI + i) * 2048 + fr);
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int j = 0; j < TJ; ++j)
          acc[i][j] = __builtin_amdgcn_mfma_f32_32x32x16_bf16(__builtin_bit_cast(bf16x8, a[i]),
                                                               __builtin_bit_cast(bf16x8, b[j]), acc[i][j], 0, 0, 0);
    }
    lds_barrier();  // stage kt's buffer is refilled by the next iteration's issue
  }
  // 32x32 accumulator layout: element e of lane l is row 8 (e / 4) + 4 (l / 32) + e % 4, column l % 32
  if (bn_part != nullptr) {
    // BatchNorm partial sums of the tile's columns over its 256 rows (rows past M
    // hold zero), in fp64: per lane over its 32 rows of each column, then the
    // other half-wave's rows, then the four row waves in a fixed order
    double sm[TJ], sq[TJ];
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      sm[j] = 0.0;
      sq[j] = 0.0;
#pragma unroll
      for (int i = 0; i < TI; ++i)
#pragma unroll
        for (int e = 0; e < 16; ++e) {
          const double v = double(acc[i][j][e]);
          sm[j] += v;
          sq[j] += v * v;
        }
      sm[j] += __shfl_xor(sm[j], 32, 64);
      sq[j] += __shfl_xor(sq[j], 32, 64);
    }
    double* red = reinterpret_cast<double*>(smem);  // [kDmaWM][2][BN]; the stages are no longer read
    if (lane < 32) {
#pragma unroll
      for (int j = 0; j < TJ; ++j) {
        const int cl = (wn * TJ + j) * 32 + lane;
        red[(wm * 2 + 0) * BN + cl] = sm[j];
        red[(wm * 2 + 1) * BN + cl] = sq[j];
      }
    }
    __syncthreads();
    if (tid < BN && n0 + tid < N) {
#pragma unroll
      for (int a = 0; a < 2; ++a) {
        double v = red[a * BN + tid];
#pragma unroll
        for (int w = 1; w < kDmaWM; ++w) v += red[(w * 2 + a) * BN + tid];
        bn_part[((m0 / BM) * 2 + a) * N + n0 + tid] = v;
      }
    }
  }
  char* Cb = reinterpret_cast<char*>(Cout) + int64_t(blockIdx.y) * split_stride * (out_bf16 ? 2 : 4);
#pragma unroll
  for (int i = 0; i < TI; ++i)
#pragma unroll
    for (int j = 0; j < TJ; ++j) {
      const int64_t col = n0 + (wn * TJ + j) * 32 + (lane & 31);
      if (col >= N) continue;
#pragma unroll
      for (int e = 0; e < 16; ++e) {
        const int64_t row = m0 + (wm * TI + i) * 32 + 8 * (e / 4) + 4 * fr_hi + (e % 4);
        if (row < M) {
          if (out_bf16)
            reinterpret_cast<uint16_t*>(Cb)[row * ldc + col] = f32_to_bf16(acc[i][j][e]);
          else
            reinterpret_cast<float*>(Cb)[row * ldc + col] = acc[i][j][e];
        }
      }
    }
}

__global__ __launch_bounds__(256) void sum_splits_kernel(const float* __restrict__ part, int splits,
                                                         int64_t stride, int64_t rows, int64_t cols,
                                                         int64_t ld_part, void* __restrict__ out,
                                                         int64_t ld_out, int out_bf16) {
  const int64_t n = rows * cols;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) {
    const int64_t r = i / cols, c = i - r * cols;
    float s = 0.f;
    for (int z = 0; z < splits; ++z) s += part[z * stride + r * ld_part + c];
    if (out_bf16)
      reinterpret_cast<uint16_t*>(out)[r * ld_out + c] = f32_to_bf16(s);
    else
      reinterpret_cast<float*>(out)[r * ld_out + c] = s;
  }
}

// Same as sum_splits_kernel, four consecutive columns per thread (16-byte
// loads); cols, ld_part, stride and ld_out are multiples of 4 and the pointers
// 16-byte aligned.
__global__ __launch_bounds__(256) void sum_splits4_kernel(const float* __restrict__ part, int splits,
                                                          int64_t stride, int64_t rows, int64_t cols,
                                                          int64_t ld_part, void* __restrict__ out,
                                                          int64_t ld_out, int out_bf16) {
  const int64_t n4 = rows * cols / 4;
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n4; i += int64_t(gridDim.x) * 256) {
    const int64_t r = (i * 4) / cols, c = i * 4 - r * cols;
    f32x4 acc = {0.f, 0.f, 0.f, 0.f};
    for (int z = 0; z < splits; ++z) acc += *reinterpret_cast<const f32x4*>(part + z * stride + r * ld_part + c);
    if (out_bf16) {
      uint16_t* o = reinterpret_cast<uint16_t*>(out) + r * ld_out + c;
      const uint32_t lo = uint32_t(f32_to_bf16(acc.x)) | (uint32_t(f32_to_bf16(acc.y)) << 16);
      const uint32_t hi = uint32_t(f32_to_bf16(acc.z)) | (uint32_t(f32_to_bf16(acc.w)) << 16);
      *reinterpret_cast<u32x2*>(o) = u32x2{lo, hi};
    } else {
      *reinterpret_cast<f32x4*>(reinterpret_cast<float*>(out) + r * ld_out + c) = acc;
    }
  }
}

// 64x64 tile transpose through LDS.  in_elem/out_elem in {2, 4}; 4 -> 2 rounds fp32 to bf16.
__global__ __launch_bounds__(256) void transpose_kernel(const void* __restrict__ in, int64_t rows, int64_t cols,
                                                        int64_t ld_in, void* __restrict__ out, int64_t ld_out,
                                                        int64_t rows_pad, int in_elem, int out_elem) {
  __shared__ float tile[64][65];
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int tx = threadIdx.x & 63, ty = threadIdx.x >> 6;
  for (int i = ty; i < 64; i += 4) {
    const int64_t r = r0 + i, c = c0 + tx;
    float v = 0.f;
    if (r < rows && c < cols) {
      if (in_elem == 2)
        v = bf16_to_f32(reinterpret_cast<const uint16_t*>(in)[r * ld_in + c]);
      else
        v = reinterpret_cast<const float*>(in)[r * ld_in + c];
    }
    tile[i][tx] = v;
  }
  __syncthreads();
  for (int i = ty; i < 64; i += 4) {
    const int64_t c = c0 + i, r = r0 + tx;  // output row c, column r
    if (c < cols && r < rows_pad) {
      const float v = tile[tx][i];
      if (out_elem == 2)
        reinterpret_cast<uint16_t*>(out)[c * ld_out + r] = f32_to_bf16(v);
      else
        reinterpret_cast<float*>(out)[c * ld_out + r] = v;
    }
  }
}

// 64x64 tile transpose of 2-byte elements with 16-byte global accesses: rows
// read 8 elements per thread, LDS tile padded by one dword per row, output rows
// written 8 elements per thread.  Needs ld_in, ld_out, cols and rows_pad
// multiples of 8 (rows in [rows, rows_pad) come out zero).
__global__ __launch_bounds__(256) void transpose16_kernel(const uint16_t* __restrict__ in, int64_t rows, int64_t cols,
                                                          int64_t ld_in, uint16_t* __restrict__ out, int64_t ld_out,
                                                          int64_t rows_pad) {
  __shared__ uint16_t tile[64][66];
  const int64_t r0 = int64_t(blockIdx.y) * 64, c0 = int64_t(blockIdx.x) * 64;
  const int t = threadIdx.x, tr = t >> 3, tc = (t & 7) * 8;
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int rr = tr + pass * 32;
    const int64_t r = r0 + rr, c = c0 + tc;
    u32x4 v = {0, 0, 0, 0};
    if (r < rows && c < cols) v = *reinterpret_cast<const u32x4*>(in + r * ld_in + c);
    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      tile[rr][tc + 2 * e] = uint16_t(w[e] & 0xFFFFu);
      tile[rr][tc + 2 * e + 1] = uint16_t(w[e] >> 16);
    }
  }
  __syncthreads();
#pragma unroll
  for (int pass = 0; pass < 2; ++pass) {
    const int oc = tr + pass * 32;  // output row = input column c0 + oc
    const int64_t orow = c0 + oc, ocol = r0 + tc;
    if (orow < cols && ocol < rows_pad) {
      uint32_t w[4];
#pragma unroll
      for (int e = 0; e < 4; ++e) w[e] = uint32_t(tile[tc + 2 * e][oc]) | (uint32_t(tile[tc + 2 * e + 1][oc]) << 16);
      *reinterpret_cast<u32x4*>(out + orow * ld_out + ocol) = u32x4{w[0], w[1], w[2], w[3]};
    }
  }
}

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = v;
}

}  // namespace

int gemm_nt_splits(int dtype, int64_t M, int64_t N, int64_t K, int cus, int max_splits) {
  if (max_splits < 1) max_splits = 1;
  if (cus < 1) cus = 256;
  if (!(dtype == kBF16 && K % 32 == 0)) {  // the 128x128 kernel, several blocks per CU
    const int64_t tiles = ((M + BM - 1) / BM) * ((N + BN - 1) / BN);
    int64_t sp = (int64_t(8) * cus + tiles - 1) / tiles;
    return int(sp < 1 ? 1 : sp > max_splits ? max_splits : sp);
  }
  // The 256x256 kernel holds one block per CU: blocks run in rounds of cus.
  // Time ~ rounds * K-slice (tile work) + the partial sums written and read
  // back (in units of one tile's K step: 256*256*2 flops at ~3 TFLOP/s per CU
  // against ~5 TB/s for the reduction).
  const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
  const double kstep_s = 256.0 * 256.0 * 2.0 / 3.0e12;
  int best = 1;
  double best_t = 0.0;
  for (int sp = 1; sp <= max_splits; ++sp) {
    const int64_t kchunk = ((K + sp - 1) / sp + 31) / 32 * 32;
    const int64_t rounds = (tiles * sp + cus - 1) / cus;
    const double t = double(rounds) * double(kchunk) * kstep_s +
                     (sp > 1 ? double(sp + 1) * double(M) * double(N) * 4.0 / 5.0e12 : 0.0);
    if (sp == 1 || t < best_t * 0.98) {
      best = sp;
      best_t = t;
    }
  }
  return best;
}

hipError_t launch_gemm_nt(hipStream_t s, int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                          int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, bool out_bf16,
                          int splits, int64_t split_stride, double* bn_part, bool* bn_done) {
  if (splits < 1) splits = 1;
  if (bn_done) *bn_done = false;
  if (dtype == kBF16 && K % 32 == 0 && M * lda * 2 < (int64_t(1) << 32) - 64 &&
      N * ldb * 2 < (int64_t(1) << 32) - 64) {
    int64_t kchunk = (K + splits - 1) / splits;
    kchunk = (kchunk + 31) / 32 * 32;
    const int64_t tiles = ((M + 255) / 256) * ((N + 255) / 256);
    const size_t lds = size_t(kDmaStages) * kDmaStage;
    static LdsLimit lim;
    const hipError_t e = lim.ensure(reinterpret_cast<const void*>(gemm_nt_dma_kernel), int(lds));
    if (e != hipSuccess) return e;
    const bool fuse_bn = bn_part != nullptr && splits == 1 && !out_bf16 && kBnRows == 256;
    hipLaunchKernelGGL(gemm_nt_dma_kernel, dim3(unsigned(tiles), unsigned(splits)), dim3(512), lds, s, M, N,
                       static_cast<const bf16_t*>(A), lda, static_cast<const bf16_t*>(B), ldb, C, ldc,
                       int(out_bf16), K, kchunk, split_stride, fuse_bn ? bn_part : nullptr);
    if (fuse_bn && bn_done) *bn_done = true;
    return hipGetLastError();
  }
  const int64_t bk = dtype == kBF16 ? 64 : 32;
  int64_t kchunk = (K + splits - 1) / splits;
  kchunk = (kchunk + bk - 1) / bk * bk;
  dim3 grid(unsigned((N + BN - 1) / BN), unsigned((M + BM - 1) / BM), unsigned(splits));
  if (dtype == kBF16)
    hipLaunchKernelGGL(gemm_nt_kernel<bf16_t>, grid, dim3(256), 0, s, M, N, K, static_cast<const bf16_t*>(A),
                       lda, static_cast<const bf16_t*>(B), ldb, C, ldc, int(out_bf16), kchunk, split_stride);
  else
    hipLaunchKernelGGL(gemm_nt_kernel<float>, grid, dim3(256), 0, s, M, N, K, static_cast<const float*>(A), lda,
                       static_cast<const float*>(B), ldb, C, ldc, int(out_bf16), kchunk, split_stride);
  return hipGetLastError();
}

hipError_t launch_sum_splits(hipStream_t s, const float* part, int splits, int64_t stride, int64_t rows,
                             int64_t cols, int64_t ld_part, void* out, int64_t ld_out, bool out_bf16) {
  const bool v4 = cols % 4 == 0 && ld_part % 4 == 0 && stride % 4 == 0 && ld_out % 4 == 0 &&
                  (reinterpret_cast<uintptr_t>(part) & 15) == 0 && (reinterpret_cast<uintptr_t>(out) & 15) == 0;
  if (v4) {
    int64_t blocks = (rows * cols / 4 + 255) / 256;
    if (blocks > 8192) blocks = 8192;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(sum_splits4_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, part, splits, stride, rows, cols,
                       ld_part, out, ld_out, int(out_bf16));
    return hipGetLastError();
  }
  int64_t blocks = (rows * cols + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(sum_splits_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, part, splits, stride, rows, cols,
                     ld_part, out, ld_out, int(out_bf16));
  return hipGetLastError();
}

hipError_t launch_transpose(hipStream_t s, const void* in, int64_t rows, int64_t cols, int64_t ld_in, void* out,
                            int64_t ld_out, int64_t rows_pad, int in_elem, int out_elem) {
  dim3 grid(unsigned((cols + 63) / 64), unsigned((rows_pad + 63) / 64));
  if (in_elem == 2 && out_elem == 2 && ld_in % 8 == 0 && ld_out % 8 == 0 && cols % 8 == 0 && rows_pad % 8 == 0) {
    hipLaunchKernelGGL(transpose16_kernel, grid, dim3(256), 0, s, static_cast<const uint16_t*>(in), rows, cols, ld_in,
                       static_cast<uint16_t*>(out), ld_out, rows_pad);
    return hipGetLastError();
  }
  hipLaunchKernelGGL(transpose_kernel, grid, dim3(256), 0, s, in, rows, cols, ld_in, out, ld_out, rows_pad,
                     in_elem, out_elem);
  return hipGetLastError();
}

hipError_t launch_fill_f32(hipStream_t s, float* p, int64_t n, float v) {
  int64_t blocks = (n + 255) / 256;
  if (blocks > 8192) blocks = 8192;
  if (blocks < 1) blocks = 1;
  hipLaunchKernelGGL(fill_f32_kernel, dim3(unsigned(blocks)), dim3(256), 0, s, p, n, v);
  return hipGetLastError();
}

}  // namespace pkm
