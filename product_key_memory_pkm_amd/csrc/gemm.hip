// Dense matrix products of the query network (steps a1 and a10):
//   forward  q_pre = x W_q^T                 (M = T,    N = h*dq, K = d)
//   backward dW_q  = dq_pre^T x              (M = h*dq, N = d,    K = T, split over K)
//            dx    = dq_pre W_q              (M = T,    N = d,    K = h*dq)
// all as C[M, N] = A[M, K] B[N, K]^T with both operands K-contiguous.
// ("Meta AI 可扩展内存层", sections 3.2 and 10.1: bias-free linear query
// projection; product-key paper summary, method details: every parameter is
// trained by back-propagation.)
//
// 128x128 output tile per 256-thread workgroup, 2x2 waves of 64x64, K staged
// through double-buffered LDS in 128-byte slices (64 bf16 or 32 fp32); bf16
// uses v_mfma_f32_16x16x32_bf16 and fp32 uses v_mfma_f32_16x16x4f32, both with
// fp32 accumulation.  The next K slice is fetched into registers while the
// current one feeds the MFMAs.  Rows padded in LDS by 16 bytes so the 16-byte
// fragment reads of 16 consecutive rows hit distinct banks.
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

__global__ void fill_f32_kernel(float* p, int64_t n, float v) {
  for (int64_t i = int64_t(blockIdx.x) * 256 + threadIdx.x; i < n; i += int64_t(gridDim.x) * 256) p[i] = v;
}

}  // namespace

hipError_t launch_gemm_nt(hipStream_t s, int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                          int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, bool out_bf16,
                          int splits, int64_t split_stride) {
  if (splits < 1) splits = 1;
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
