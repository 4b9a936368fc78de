// Host-side launchers of the PKM kernels (internal to the library).
#pragma once

#include <hip/hip_runtime.h>
#include <stddef.h>
#include <stdint.h>

#include <atomic>

namespace pkm {

// Raises one kernel's dynamic LDS limit (hipFuncAttributeMaxDynamicSharedMemorySize)
// to `bytes` the first time it is launched on each device: devices 0..63 are
// remembered, others set it on every launch.  Safe to call from several host
// threads (two first launches may both set it, which is harmless).
class LdsLimit {
 public:
  hipError_t ensure(const void* fn, int bytes) {
    int dev = 0;
    hipError_t e = hipGetDevice(&dev);
    if (e != hipSuccess) return e;
    const uint64_t bit = dev >= 0 && dev < 64 ? uint64_t(1) << dev : 0;
    if (bit != 0 && (done_.load(std::memory_order_acquire) & bit) != 0) return hipSuccess;
    e = hipFuncSetAttribute(fn, hipFuncAttributeMaxDynamicSharedMemorySize, bytes);
    if (e == hipSuccess) done_.fetch_or(bit, std::memory_order_acq_rel);
    return e;
  }

 private:
  std::atomic<uint64_t> done_{0};
};

constexpr int kF32 = 0;
constexpr int kBF16 = 1;

// a6: y[t] = sum_r w[t, r] V[idx[t, r]] over R = h*k rows per token.
// fp8_values: rows of [16-byte header (fp32 scale), d_value E4M3 codes].
// resid (storage values only; may be null): resid[t] = y[t] as stored - target[t],
// rounded to the storage type.
hipError_t launch_gather(hipStream_t s, int dtype, const int32_t* idx, const float* w, const void* V,
                         void* y, int64_t ntok, int R, int d_value, bool fp8_values,
                         const void* target = nullptr, void* resid = nullptr);
// a5 + a6 in one launch (the forward): merge_softmax's idx and w for every
// (token, head) and launch_gather's y from them, bit-identical to the two
// launches.  Supported when merge_gather_supported (k divides 64, rows of at
// most 256 16-byte vectors, storage-dtype values); else hipErrorInvalidValue.
bool merge_gather_supported(int dtype, int k, int d_value, bool fp8_values);
// target, resid (both or neither): also the residual resid = y - target [ntok,
// d_value], as launch_gather writes it.
hipError_t launch_merge_gather(hipStream_t s, int dtype, const int32_t* sub_idx, const float* sub_score, int64_t ntok,
                               int heads, int k, int nk2, float inv_tau, int32_t* idx, float* w, const void* V,
                               void* y, int d_value, bool fp8_values, const void* target = nullptr,
                               void* resid = nullptr);
// fp8 value rows from rows in the storage dtype (d_value % 16 == 0).
hipError_t launch_quantize_fp8(hipStream_t s, int dtype, const void* src, int64_t rows, int d_value, void* dst);

// a3 + a4: per (token, head, half) scores against the half's sub-keys and top-k.
// packed: score_topk_packed_bytes of scratch for the repacked sub-keys.
// Returns hipErrorInvalidValue when the shape does not fit the kernel's LDS plan.
bool score_topk_supported(int dtype, int half, int nkeys);
size_t score_topk_packed_bytes(int dtype, int heads, int half, int nk, int nk2);
// idw: scores -log |q_half - c| (squared distance floored at 1e-12) instead of q_half . c.
// list: score_select_list_bytes(ntok, heads) of scratch (the rows the
// register-resident kernel hands to its exact second launch).
hipError_t launch_score_topk(hipStream_t s, int dtype, const void* q, int64_t ntok, int heads, int dq,
                             const void* C, const void* Cp, int nk, int nk2, int k, int32_t* sub_idx,
                             float* sub_score, void* packed, bool idw, void* list);
// The same step for bf16 codebooks of 257-2048 sub-keys with the scores of a
// token tile kept in registers (launch_score_topk takes it where supported).
bool score_select_supported(int dtype, int half, int nk, int nk2, int k, bool idw);
size_t score_select_packed_bytes(int heads, int half, int nk, int nk2);
size_t score_select_list_bytes(int64_t ntok, int heads);
hipError_t launch_score_select(hipStream_t s, const void* q, int64_t ntok, int heads, int dq, const void* C,
                               const void* Cp, int nk, int nk2, int k, int32_t* sub_idx, float* sub_score,
                               void* packed, void* list);

// a5: k x k candidates -> top-k -> softmax, per (token, head).
// group_items > 0: item i's rows are offset by ((i / group_items) % group_count) * group_rows
// (consecutive groups of items address consecutive tables of group_rows rows,
// starting over at the first table every group_count groups).
hipError_t launch_merge_softmax(hipStream_t s, const int32_t* sub_idx, const float* sub_score,
                                int64_t nitems, int k, int nk2, float inv_tau, int32_t* idx, float* w,
                                float* score, int64_t group_items = 0, int64_t group_rows = 0,
                                int64_t group_count = 1);

// C[M, N] = A[M, K] * B[N, K]^T; A, B storage dtype, C fp32 (or bf16 when out_bf16).
// splits > 1: blockIdx.z handles a slice of K and writes C + z * split_stride.
// bn_part (may be null; fp32 output, one split only): also the BatchNorm
// partial sums of C's columns over row blocks of kBnRows, in the layout of
// launch_bn_partials, when the kernel taking this shape can give them; then
// *bn_done is set (else left false and the caller runs launch_bn_partials).
hipError_t launch_gemm_nt(hipStream_t s, int dtype, int64_t M, int64_t N, int64_t K, const void* A,
                          int64_t lda, const void* B, int64_t ldb, void* C, int64_t ldc, bool out_bf16,
                          int splits, int64_t split_stride, double* bn_part = nullptr, bool* bn_done = nullptr);
// Split-K count for launch_gemm_nt on a device with cus compute units: whole
// rounds of resident blocks, the partial-sum traffic counted against it.
int gemm_nt_splits(int dtype, int64_t M, int64_t N, int64_t K, int cus, int max_splits);
// out[i] = sum_z part[z * stride + i] for i < n (fixed order), optional bf16 output.
hipError_t launch_sum_splits(hipStream_t s, const float* part, int splits, int64_t stride, int64_t rows,
                             int64_t cols, int64_t ld_part, void* out, int64_t ld_out, bool out_bf16);
// out[c, r] = in[r, c] for r < rows, c < cols; zero for r in [rows, rows_pad).
// Element size 2 or 4 bytes; in_f32_to_bf16 converts fp32 input to bf16 output.
hipError_t launch_transpose(hipStream_t s, const void* in, int64_t rows, int64_t cols, int64_t ld_in,
                            void* out, int64_t ld_out, int64_t rows_pad, int in_elem, int out_elem);

// a2: BatchNorm.
// Per-block partial sums (fp64) of q_pre columns over row blocks of kBnRows.
constexpr int kBnRows = 256;
hipError_t launch_bn_partials(hipStream_t s, const float* q_pre, int64_t ntok, int F, double* part);
hipError_t launch_bn_finalize(hipStream_t s, const double* part, int nblk, int64_t ntok, int F, float eps,
                              float* mean, float* rstd);
hipError_t launch_bn_apply(hipStream_t s, int dtype, const float* q_pre, int64_t ntok, int F,
                           const float* mean, const float* rstd, const float* gamma, const float* beta,
                           void* q);
// a10: partial sums of dq and dq * xhat per column block.
hipError_t launch_bn_bwd_partials(hipStream_t s, const float* dq, const float* q_pre, const float* mean,
                                  const float* rstd, int64_t ntok, int F, double* part);
hipError_t launch_bn_bwd_finalize(hipStream_t s, const double* part, int nblk, int F, const float* gamma,
                                  float* dgamma, float* dbeta, float* coef);
// dq_pre = gamma*rstd*(dq - dbeta/T - xhat*dgamma/T); written row-major (out_rm,
// [ntok, ld_rm]) and transposed (out_tr, [F, ld_tr], zero in columns [ntok, rows_pad)),
// each as fp32 or bf16 per dtype.
hipError_t launch_bn_bwd_apply(hipStream_t s, int dtype, const float* dq, const float* q_pre,
                               const float* mean, const float* rstd, const float* gamma,
                               const float* dgamma, const float* dbeta, int64_t ntok, int F, bool bn,
                               void* out_rm, int64_t ld_rm, void* out_tr, int64_t ld_tr, int64_t rows_pad);

// Stable radix sort by key of n keys (< 2^key_bits) paired with their indices 0..n-1.
// keys_in is read only; the passes ping-pong between (k0, v0) and (k1, v1) and
// *result_in_1 tells which pair holds the sorted result.
size_t radix_sort_temp_bytes(int64_t n);
hipError_t launch_radix_sort_from(hipStream_t s, const uint32_t* keys_in, uint32_t* k0, int32_t* v0,
                                  uint32_t* k1, int32_t* v1, int64_t n, int key_bits, void* temp,
                                  bool* result_in_1);
// Scratch of launch_segments over n sorted keys (the per-block segment counts).
size_t scan_temp_bytes(int64_t n);

// The value gradient's long-run plan: every run of more than kVgChunk lookups
// of one row is cut into chunks, listed as (run, chunk) in chunk_list and
// (run, first chunk slot) in long_list; counts = {chunks, long runs}.  The
// lists live in the value gradient's aux buffer.
constexpr int kVgChunk = 256;
struct VgPlan {
  uint32_t* counts;
  int2* chunk_list;
  int2* long_list;
};
VgPlan value_grad_plan(void* aux, int64_t nitems, int d_value);

// Both of the above for n <= kSmallSortMax pairs in one launch: keys_in (< 2^key_bits)
// stably sorted into keys_out with their indices in vals_out, and the segment
// table (seg_start, touched (may be null), count) of the sorted keys; plan
// (may be null): also the value gradient's long-run plan of those segments.
constexpr int kSmallSortMax = 8192;
hipError_t launch_sort_segments_small(hipStream_t s, const uint32_t* keys_in, int64_t n, int key_bits,
                                      uint32_t* keys_out, int32_t* vals_out, int32_t* seg_start, int32_t* touched,
                                      int64_t* count, const VgPlan* plan = nullptr);
// The same for n pairs in `groups` equal groups of at most kSmallSortMax, every
// key of a group below every key of the next (groups <= kSortGroupsMax): one
// workgroup per group, then one that joins their segment tables and builds
// the plan.  key_bits: the bits in which keys of one group differ (from bit 0).
// temp: sort_groups_temp_bytes(n).
constexpr int kSortGroupsMax = 1024;
size_t sort_groups_temp_bytes(int64_t n);
// The groups left apart (no key order between them needed): group g of the
// n / groups pairs [g n/groups, (g+1) n/groups) gets its own segment table at
// seg_g + g (n/groups + 1) (positions global), count at cnt_g[g] and long-run
// plan group_plan(plans, g); plans holds groups * group_plan_stride() bytes.
size_t group_plan_stride();
VgPlan group_plan(void* plans, int g);
hipError_t launch_sort_segments_separate(hipStream_t s, const uint32_t* keys_in, int64_t n, int groups, int key_bits,
                                         uint32_t* keys_out, int32_t* vals_out, int32_t* seg_g, int64_t* cnt_g,
                                         void* plans);
// Joins `groups` consecutive separate tables (seg_g, cnt_g pointing at the
// first; every key of a group below every key of the next) into seg_start /
// count, with end_pos the position after the last group's last pair, and
// lists their long runs in plan (its counts zeroed here first).
hipError_t launch_join_groups(hipStream_t s, const int32_t* seg_g, const int64_t* cnt_g, int groups, int n_per,
                              int64_t end_pos, int32_t* seg_start, int64_t* count, const VgPlan* plan);
hipError_t launch_sort_segments_grouped(hipStream_t s, const uint32_t* keys_in, int64_t n, int groups,
                                        int key_bits, uint32_t* keys_out, int32_t* vals_out, int32_t* seg_start,
                                        int32_t* touched, int64_t* count, const VgPlan* plan, void* temp);

// Segments of a sorted key array: seg_start[u] for every distinct key run, and
// count (device int64).  Also touched[u] = key of run u (may be null).
// seg_start needs room for count + 1 entries (the last one is n).
hipError_t launch_segments(hipStream_t s, const uint32_t* sorted_keys, int64_t n, int32_t* seg_start,
                           int32_t* touched, int64_t* count, void* scan_temp);

// a7 + a8: per touched row, dw for every lookup of it and the row's dV.  Rows
// with more lookups than a chunk are split over several waves; aux (of
// value_grad_aux_bytes) holds their lists and partial sums.  plan_ready: the
// long-run plan is already in aux (launch_sort_segments_small wrote it).
// adam != null: no dV; every touched row's gradient takes an Adam step on
// (V, m, v) instead (V is then the same buffer as adam->V, updated in place).
struct VgAdam {
  void* V;
  float* m;
  float* v;
  float beta1, beta2, eps;
  float step_size;     // lr / (1 - beta1^step); with sgd the learning rate
  float inv_sqrt_bc2;  // 1 / sqrt(1 - beta2^step)
  int sgd;             // 1: plain step V -= step_size * g (m, v unused)
  // moments in a pool of slots (null: m, v are dense [rows, d_value] tables):
  // slot[r] = -1 (no moments: the row is not stepped), s (moments in pool row
  // s), or -2 - s (slot s handed out in this call: zero moments, then s stored)
  int32_t* slot;
  int64_t capacity;
  int64_t* n_used;  // slots handed out so far (device)
};
// Bytes of one fp8 value row of nvec 16-code vectors: the 16-byte header and
// the codes, rounded up to whole 128-byte lines.
__host__ __device__ constexpr size_t fp8_row_bytes(int nvec) {
  return (size_t(nvec) * 16 + 16 + 127) / 128 * 128;
}
// Hands out pool slots to the touched rows that have none (slot[r] == -1), in
// ascending row order from *n_used; a slot at or past capacity is refused (the
// entry stays -1) but counted in *n_used.  tmp: row_state_temp_bytes().
size_t row_state_temp_bytes();
hipError_t launch_row_state_assign(hipStream_t s, const int32_t* touched, const int64_t* n_touched, int32_t* slot,
                                   int64_t capacity, int64_t* n_used, void* tmp);
size_t value_grad_aux_bytes(int64_t nitems, int d_value);
hipError_t launch_value_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg,
                             int64_t nitems, const uint32_t* sorted_rows, const int32_t* sorted_c,
                             const float* w, const void* dY, const void* V, float* dV, float* dw,
                             int R, int d_value, bool accumulate, void* aux, const VgAdam* adam = nullptr,
                             bool plan_ready = false, const VgPlan* plan = nullptr);

// a7 + a9: per (token, head) softmax backward, dq from the distinct selected
// sub-keys, and per slot the sub-key sort key (h*|C|+i / h*|C'|+j, or the
// sentinel h*|C| / h*|C'| for a repeated sub-key) with the summed coefficient.
hipError_t launch_softmax_bwd_dq(hipStream_t s, int dtype, const int32_t* idx, const float* w,
                                 const float* dw, const void* C, const void* Cp, int64_t ntok, int heads,
                                 int dq, int k, int nk, int nk2, float inv_tau, float* dq_out, uint32_t* key1,
                                 float* coef1, uint32_t* key2, float* coef2);
// dC[key] = sum over its sorted entries of coef[c] * q_half[t(c), h], one block per
// sub-key, sub-keys with more entries than a chunk split over several blocks;
// aux (of subkey_grad_aux_bytes) holds their lists and partial sums.  Sub-keys
// without entries are left alone (the caller clears dC first).
size_t subkey_grad_aux_bytes(int64_t nitems, int dq);
hipError_t launch_subkey_grad(hipStream_t s, int dtype, const int32_t* seg_start, const int64_t* nseg,
                              int64_t nsub, int64_t nitems, const uint32_t* sorted_keys, const int32_t* sorted_c,
                              const float* coef, const void* q, int heads, int dq, int k, int half_sel,
                              int nkeys, float* dC, void* aux);

hipError_t launch_fill_f32(hipStream_t s, float* p, int64_t n, float v);

// Monitoring signals of a selection (idx, w [ntok, heads, k]): sub-key hit
// counts, slots in use (all heads, then per head), entropy per (t, h) (may be
// null) and its fp64 sum (may be null).  ws: diagnostics_ws_bytes.
size_t diagnostics_ws_bytes(int64_t ntok, int heads, int64_t nrows);
hipError_t launch_diagnostics(hipStream_t s, const int32_t* idx, const float* w, int64_t ntok, int heads, int k,
                              int nk, int nk2, int32_t* hits_c, int32_t* hits_cp, int64_t* used, float* entropy,
                              double* entropy_sum, void* ws);

}  // namespace pkm
