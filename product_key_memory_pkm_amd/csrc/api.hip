// C ABI of the product-key memory lookup: argument checks, workspace layout and
// the order of kernel launches on the caller's stream.  The steps follow
// "Meta AI 可扩展内存层" (sections 3.2, 4.3, 4.5, 5.3, 6.1, 9.2, 10.1) and the
// product-key paper summary (method details, key results); see include/pkm.h.
#include <stdarg.h>
#include <stdio.h>

#include <algorithm>
#include <cmath>
#include <mutex>
#include <new>
#include <string>

#include "kernels.h"
#include "pkm.h"

using namespace pkm;

struct pkm_handle_s {
  pkm_config cfg;
  int half;   // dq / 2
  int F;      // heads * dq
  int elem;   // bytes per storage element
  int row_bits;
  // second stream of pkm_backward (sub-key gradients beside the projection
  // gradients), with its fork/join events; absent (null) if creation failed
  int device;
  int cus;  // compute units of the device (split-K sizing)
  hipStream_t side;
  hipEvent_t fork, join;
  std::mutex side_mu;  // one backward at a time enqueues on the side stream
};

namespace {

thread_local std::string g_err;

pkm_status fail(pkm_status s, const char* fmt, ...) {
  char buf[512];
  va_list ap;
  va_start(ap, fmt);
  vsnprintf(buf, sizeof buf, fmt, ap);
  va_end(ap);
  g_err = buf;
  return s;
}

pkm_status hip_check(hipError_t e, const char* what) {
  if (e != hipSuccess) return fail(PKM_ERR_HIP, "%s: %s", what, hipGetErrorString(e));
  return PKM_OK;
}

#define PKM_TRY(x)                    \
  do {                                \
    pkm_status _st = (x);             \
    if (_st != PKM_OK) return _st;    \
  } while (0)
#define PKM_HIP(call, what) PKM_TRY(hip_check((call), what))

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }

pkm_status need(const void* p, const char* name) {
  if (p == nullptr) return fail(PKM_ERR_INVALID_ARG, "%s is NULL", name);
  if (!aligned16(p)) return fail(PKM_ERR_INVALID_ARG, "%s is not 16-byte aligned", name);
  return PKM_OK;
}

size_t al(size_t x) { return (x + 255) & ~size_t(255); }

int64_t round_up(int64_t a, int64_t b) { return (a + b - 1) / b * b; }

// Workspace regions.  Forward and backward layouts start at offset 0 and the
// backward layout never needs the forward's regions, so one buffer of the
// larger size serves both.
struct FwdLayout {
  size_t sub_idx, sub_score, bn_part, keys, sel_list, total;
};
struct BwdLayout {
  size_t k0, v0, k1, v1, sort_tmp, grp, key1, key2, seg, scan_tmp, nseg, dw, ds, coef2, dq, bn_part,
      dqpre, dqpre_t, x_t, wq_t, split, aux, rstate, total;
  int splits;
  int64_t tpad;
  // leading dimensions of the GEMM operands written here: 64 elements past a
  // multiple of 64 so that a tile's rows do not all start at the same offset
  // modulo a large power of two
  int64_t ldt;  // dqpre_t, x_t: [F | d_in, ldt], columns [0, tpad) used
  int64_t ldf;  // dqpre: [T, ldf]; wq_t: [d_in, ldf]
};

FwdLayout fwd_layout(const pkm_handle_s* h, int64_t T) {
  const pkm_config& c = h->cfg;
  FwdLayout L{};
  size_t o = 0;
  const size_t nsub = size_t(T) * c.heads * 2 * c.topk;
  L.sub_idx = o;  o += al(nsub * 4);
  L.sub_score = o; o += al(nsub * 4);
  const size_t nblk = size_t((T + kBnRows - 1) / kBnRows);
  L.bn_part = o;  o += al(nblk * 2 * h->F * sizeof(double));
  L.keys = o;     o += al(score_topk_packed_bytes(c.dtype, c.heads, h->half, c.n_keys, c.n_keys2));
  L.sel_list = o; o += al(score_select_list_bytes(T, c.heads));
  L.total = o;
  return L;
}

int dwq_splits(const pkm_handle_s* h, int64_t tpad) {
  int64_t maxs = tpad / 256 > 1 ? tpad / 256 : 1;
  if (maxs > 32) maxs = 32;
  return gemm_nt_splits(h->cfg.dtype, h->F, h->cfg.d_in, tpad, h->cus, int(maxs));
}

BwdLayout bwd_layout(const pkm_handle_s* h, int64_t T) {
  const pkm_config& c = h->cfg;
  BwdLayout L{};
  const size_t N = size_t(T) * c.heads * c.topk;
  size_t o = 0;
  L.k0 = o; o += al(N * 4);
  L.v0 = o; o += al(N * 4);
  L.k1 = o; o += al(N * 4);
  L.v1 = o; o += al(N * 4);
  L.sort_tmp = o; o += al(radix_sort_temp_bytes(int64_t(N)));
  L.grp = o; o += al(sort_groups_temp_bytes(int64_t(N)));  // per-group segment tables of a grouped sort
  L.key1 = o; o += al(N * 4);  // per-slot sub-key sort keys of the two halves
  L.key2 = o; o += al(N * 4);
  L.seg = o; o += al((N + 1) * 4);
  L.scan_tmp = o; o += al(256 + scan_temp_bytes(int64_t(N)));
  L.nseg = o; o += al(4 * sizeof(int64_t));
  L.dw = o; o += al(N * 4);
  L.ds = o; o += al(N * 4);
  L.coef2 = o; o += al(N * 4);
  L.dq = o; o += al(size_t(T) * h->F * 4);
  const size_t nblk = size_t((T + kBnRows - 1) / kBnRows);
  L.bn_part = o; o += al(nblk * 2 * h->F * sizeof(double));
  L.tpad = round_up(T, 64);
  L.ldt = L.tpad + 64;
  L.ldf = round_up(h->F, 64) + 64;
  L.dqpre = o; o += al(size_t(T) * L.ldf * h->elem);
  L.dqpre_t = o; o += al(size_t(h->F) * L.ldt * h->elem);
  L.x_t = o; o += al(size_t(c.d_in) * L.ldt * h->elem);
  L.wq_t = o; o += al(size_t(c.d_in) * L.ldf * h->elem);
  L.splits = dwq_splits(h, L.tpad);
  L.split = o; o += al(size_t(L.splits) * h->F * c.d_in * 4);
  // long-run lists and partial sums of the value and sub-key gradients (used one after the other)
  L.aux = o; o += al(std::max(value_grad_aux_bytes(int64_t(N), c.d_value), subkey_grad_aux_bytes(int64_t(N), c.d_query)));
  L.rstate = o; o += al(row_state_temp_bytes());  // slot hand-out of the Adam moment pool
  L.total = o;
  return L;
}

// FwPKM memorization chunk: the forward's and the backward's regions (used one
// after the other), then the residual e [T, d_value] (storage dtype), the
// touched rows and their count.
struct ChunkLayout {
  size_t e, touched, n_touched, plans, total;
};

ChunkLayout chunk_layout(const pkm_handle_s* h, int64_t T) {
  const size_t N = size_t(T) * h->cfg.heads * h->cfg.topk;
  ChunkLayout L{};
  size_t o = std::max(fwd_layout(h, T).total, bwd_layout(h, T).total);
  L.e = o; o += al(size_t(T) * h->cfg.d_value * h->elem);
  L.touched = o; o += al(N * 4);
  L.n_touched = o; o += al(sizeof(int64_t));
  L.plans = o; o += al(size_t(kSortGroupsMax) * group_plan_stride());  // pkm_fwpkm_chunks' per-call plans
  L.total = o;
  return L;
}

size_t ws_size(const pkm_handle_s* h, int64_t T, int with_backward) {
  const size_t f = fwd_layout(h, T).total;
  if (with_backward == PKM_WS_FORWARD) return f;
  if (with_backward == PKM_WS_FWPKM_CHUNK) return chunk_layout(h, T).total;
  const size_t b = std::max(bwd_layout(h, T).total,
                            diagnostics_ws_bytes(T, h->cfg.heads, int64_t(h->cfg.n_keys) * h->cfg.n_keys2));
  return f > b ? f : b;
}

pkm_status check_handle(pkm_handle_t h) {
  if (h == nullptr) return fail(PKM_ERR_INVALID_ARG, "handle is NULL");
  return PKM_OK;
}

// Entry points that read V in the backward need it in the storage dtype.
pkm_status need_storage_values(pkm_handle_t h) {
  if (h->cfg.value_format == PKM_VALUES_FP8)
    return fail(PKM_ERR_UNSUPPORTED, "fp8 values are a forward format; the backward needs V in the storage dtype");
  return PKM_OK;
}

// The gradients through the scores are those of the dot product.
pkm_status need_dot_scores(pkm_handle_t h) {
  if (h->cfg.score_fn != PKM_SCORE_DOT)
    return fail(PKM_ERR_UNSUPPORTED, "the sub-key and query gradients are implemented for dot-product scores only");
  return PKM_OK;
}

pkm_status check_T(const pkm_handle_s* h, int64_t T) {
  if (T < 0) return fail(PKM_ERR_INVALID_ARG, "T = %lld is negative", (long long)T);
  const int64_t N = T * h->cfg.heads * h->cfg.topk;
  if (N > (int64_t(1) << 26))
    return fail(PKM_ERR_UNSUPPORTED, "T*heads*topk = %lld exceeds 2^26 lookups per call", (long long)N);
  return PKM_OK;
}

pkm_status check_ws(const pkm_handle_s* h, int64_t T, int with_backward, const void* ws, size_t ws_bytes) {
  const size_t want = ws_size(h, T, with_backward);
  if (ws == nullptr) return fail(PKM_ERR_WORKSPACE, "workspace is NULL (%zu bytes needed)", want);
  if (!aligned16(ws)) return fail(PKM_ERR_WORKSPACE, "workspace is not 16-byte aligned");
  if (ws_bytes < want) return fail(PKM_ERR_WORKSPACE, "workspace of %zu bytes, %zu needed", ws_bytes, want);
  return PKM_OK;
}

template <typename P>
P* at(void* ws, size_t off) {
  return reinterpret_cast<P*>(static_cast<char*>(ws) + off);
}

hipStream_t as_stream(void* s) { return static_cast<hipStream_t>(s); }

// ---- step groups shared by the full calls and the stage entry points ----

pkm_status run_query(const pkm_handle_s* h, hipStream_t s, int64_t T, const void* x, const void* Wq,
                     const float* gamma, const float* beta, const pkm_saved* sv, void* ws) {
  const pkm_config& c = h->cfg;
  const FwdLayout L = fwd_layout(h, T);
  const bool bn = c.bn == PKM_BN_BATCH;
  double* part = at<double>(ws, L.bn_part);
  bool partials_done = false;  // the projection's epilogue may give the BatchNorm partial sums
  PKM_HIP(launch_gemm_nt(s, c.dtype, T, h->F, c.d_in, x, c.d_in, Wq, c.d_in, sv->q_pre, h->F, false, 1, 0,
                         bn ? part : nullptr, &partials_done),
          "projection GEMM");
  if (bn) {
    const int nblk = int((T + kBnRows - 1) / kBnRows);
    if (!partials_done) PKM_HIP(launch_bn_partials(s, sv->q_pre, T, h->F, part), "BatchNorm partial sums");
    PKM_HIP(launch_bn_finalize(s, part, nblk, T, h->F, c.bn_eps, sv->bn_mean, sv->bn_rstd), "BatchNorm finalize");
    PKM_HIP(launch_bn_apply(s, c.dtype, sv->q_pre, T, h->F, sv->bn_mean, sv->bn_rstd, gamma, beta, sv->q),
            "BatchNorm apply");
  } else {
    PKM_HIP(launch_bn_apply(s, c.dtype, sv->q_pre, T, h->F, nullptr, nullptr, nullptr, nullptr, sv->q),
            "query cast");
  }
  return PKM_OK;
}

pkm_status run_score(const pkm_handle_s* h, hipStream_t s, int64_t T, const void* q, const void* C, const void* Cp,
                     int32_t* sub_idx, float* sub_score, void* ws) {
  const pkm_config& c = h->cfg;
  const FwdLayout L = fwd_layout(h, T);
  PKM_HIP(launch_score_topk(s, c.dtype, q, T, c.heads, c.d_query, C, Cp, c.n_keys, c.n_keys2, c.topk, sub_idx,
                            sub_score, at<void>(ws, L.keys), c.score_fn == PKM_SCORE_IDW, at<void>(ws, L.sel_list)),
          "sub-key scoring / top-k");
  return PKM_OK;
}

pkm_status run_merge(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* sub_idx, const float* sub_score,
                     int32_t* idx, float* w, float* score, int64_t group_tokens = 0, int64_t group_count = 1) {
  const pkm_config& c = h->cfg;
  PKM_HIP(launch_merge_softmax(s, sub_idx, sub_score, T * c.heads, c.topk, c.n_keys2, 1.0f / c.temperature, idx, w,
                               score, group_tokens * c.heads, int64_t(c.n_keys) * c.n_keys2, group_count),
          "candidate merge / softmax");
  return PKM_OK;
}

pkm_status run_gather(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* idx, const float* w,
                      const void* V, void* y) {
  const pkm_config& c = h->cfg;
  PKM_HIP(launch_gather(s, c.dtype, idx, w, V, y, T, c.heads * c.topk, c.d_value, c.value_format == PKM_VALUES_FP8),
          "value gather-sum");
  return PKM_OK;
}

// bits < 0: the handle's row ids; otherwise keys below 2^bits (several tables).
int row_sort_passes(const pkm_handle_s* h, int bits = -1) {
  const int p = ((bits < 0 ? h->row_bits : bits) + 7) / 8;
  return p < 1 ? 1 : p;
}

// Lookups that come in `groups` equal groups addressing ascending, disjoint
// row ranges (the streams of a memorization batch) too many for one workgroup
// but few enough per group are sorted a workgroup per group.
bool grouped_sort(int64_t N, int groups) {
  return groups > 1 && N > kSmallSortMax && N % groups == 0 && N / groups <= kSmallSortMax &&
         groups <= kSortGroupsMax;
}

// Grouping of the lookups by row.  The sorted (row, lookup) pairs land in
// (k0, v0) or (k1, v1) depending on the number of radix passes; a small batch
// is sorted and segmented in one workgroup, straight into the same place.
pkm_status run_row_groups(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* idx, int32_t* touched,
                          int64_t* n_touched, void* ws, int bits = -1, int groups = 1) {
  const pkm_config& c = h->cfg;
  const BwdLayout L = bwd_layout(h, T);
  const int64_t N = T * c.heads * c.topk;
  const int key_bits = bits < 0 ? h->row_bits : bits;
  if (grouped_sort(N, groups)) {  // each group's keys differ only in the handle's row bits
    const bool out1 = row_sort_passes(h, key_bits) % 2 == 0;
    const VgPlan plan = value_grad_plan(at<void>(ws, L.aux), N, c.d_value);
    PKM_HIP(launch_sort_segments_grouped(s, reinterpret_cast<const uint32_t*>(idx), N, groups, h->row_bits,
                                         at<uint32_t>(ws, out1 ? L.k1 : L.k0), at<int32_t>(ws, out1 ? L.v1 : L.v0),
                                         at<int32_t>(ws, L.seg), touched, n_touched, &plan, at<void>(ws, L.grp)),
            "row sort, segments and long-run plan (a workgroup per group)");
    return PKM_OK;
  }
  if (N <= kSmallSortMax) {
    const bool out1 = row_sort_passes(h, key_bits) % 2 == 0;
    const VgPlan plan = value_grad_plan(at<void>(ws, L.aux), N, c.d_value);
    PKM_HIP(launch_sort_segments_small(s, reinterpret_cast<const uint32_t*>(idx), N, key_bits,
                                       at<uint32_t>(ws, out1 ? L.k1 : L.k0), at<int32_t>(ws, out1 ? L.v1 : L.v0),
                                       at<int32_t>(ws, L.seg), touched, n_touched, &plan),
            "row sort, segments and long-run plan (one workgroup)");
    return PKM_OK;
  }
  bool in1 = false;
  PKM_HIP(launch_radix_sort_from(s, reinterpret_cast<const uint32_t*>(idx), at<uint32_t>(ws, L.k0),
                                 at<int32_t>(ws, L.v0), at<uint32_t>(ws, L.k1), at<int32_t>(ws, L.v1), N, key_bits,
                                 at<void>(ws, L.sort_tmp), &in1),
          "row sort");
  const uint32_t* sk = at<uint32_t>(ws, in1 ? L.k1 : L.k0);
  PKM_HIP(launch_segments(s, sk, N, at<int32_t>(ws, L.seg), touched, n_touched, at<void>(ws, L.scan_tmp)),
          "row segments");
  return PKM_OK;
}

pkm_status run_value_grad_grouped(const pkm_handle_s* h, hipStream_t s, int64_t T, const float* w, const void* dY,
                                  const void* V, float* dV, float* dw, const int64_t* n_touched, void* ws,
                                  const VgAdam* adam = nullptr, int bits = -1, int groups = 1) {
  const pkm_config& c = h->cfg;
  const BwdLayout L = bwd_layout(h, T);
  const int64_t N = T * c.heads * c.topk;
  const bool in1 = row_sort_passes(h, bits) % 2 == 0;  // passes alternate (k0,v0), (k1,v1), ...
  const uint32_t* sk = at<uint32_t>(ws, in1 ? L.k1 : L.k0);
  const int32_t* sv = at<int32_t>(ws, in1 ? L.v1 : L.v0);
  // a grouping made in one workgroup (or one per group) came with the long-run plan in aux
  PKM_HIP(launch_value_grad(s, c.dtype, at<int32_t>(ws, L.seg), n_touched, N, sk, sv, w, dY, V, dV, dw,
                            c.heads * c.topk, c.d_value, c.accumulate_dv != 0, at<void>(ws, L.aux), adam,
                            N <= kSmallSortMax || grouped_sort(N, groups)),
          adam ? "value gradient with Adam step" : "value gradient");
  return PKM_OK;
}

pkm_status run_value_grad(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* idx, const float* w,
                          const void* dY, const void* V, float* dV, int32_t* touched, int64_t* n_touched, float* dw,
                          void* ws, const VgAdam* adam = nullptr, int bits = -1, int groups = 1) {
  PKM_TRY(run_row_groups(h, s, T, idx, touched, n_touched, ws, bits, groups));
  if (adam && adam->slot) {
    PKM_HIP(launch_row_state_assign(s, touched, n_touched, adam->slot, adam->capacity, adam->n_used,
                                    at<void>(ws, bwd_layout(h, T).rstate)),
            "slot hand-out of the moment pool");
  }
  return run_value_grad_grouped(h, s, T, w, dY, V, dV, dw, n_touched, ws, adam, bits, groups);
}

// Adam hyper-parameters -> the kernel's constants (bias corrections in double).
pkm_status adam_args(const pkm_adam* hp, void* V, float* m, float* v, VgAdam* out) {
  if (hp == nullptr) return fail(PKM_ERR_INVALID_ARG, "adam is NULL");
  if (!(std::isfinite(hp->lr) && hp->lr >= 0.f)) return fail(PKM_ERR_INVALID_ARG, "adam.lr must be finite and >= 0");
  if (!(hp->beta1 >= 0.f && hp->beta1 < 1.f)) return fail(PKM_ERR_INVALID_ARG, "adam.beta1 must lie in [0, 1)");
  if (!(hp->beta2 >= 0.f && hp->beta2 < 1.f)) return fail(PKM_ERR_INVALID_ARG, "adam.beta2 must lie in [0, 1)");
  if (!(std::isfinite(hp->eps) && hp->eps > 0.f)) return fail(PKM_ERR_INVALID_ARG, "adam.eps must be finite and > 0");
  if (hp->step < 1) return fail(PKM_ERR_INVALID_ARG, "adam.step must be >= 1");
  const double bc1 = 1.0 - std::pow(double(hp->beta1), double(hp->step));
  const double bc2 = 1.0 - std::pow(double(hp->beta2), double(hp->step));
  out->V = V;
  out->m = m;
  out->v = v;
  out->beta1 = hp->beta1;
  out->beta2 = hp->beta2;
  out->eps = hp->eps;
  out->step_size = float(double(hp->lr) / bc1);
  out->inv_sqrt_bc2 = float(1.0 / std::sqrt(bc2));
  out->sgd = 0;
  out->slot = nullptr;
  out->capacity = 0;
  out->n_used = nullptr;
  return PKM_OK;
}

// adam_args with the moments in the slot pool of `st`.
pkm_status adam_rows_args(const pkm_handle_s* h, const pkm_adam* hp, void* V, const pkm_adam_rows* st, VgAdam* out) {
  if (st == nullptr) return fail(PKM_ERR_INVALID_ARG, "state is NULL");
  PKM_TRY(need(st->slot, "state.slot"));
  if (st->capacity != 0 || st->m != nullptr) PKM_TRY(need(st->m, "state.m"));  // a pool of no rows is never read
  if (st->capacity != 0 || st->v != nullptr) PKM_TRY(need(st->v, "state.v"));
  if (st->n_used == nullptr) return fail(PKM_ERR_INVALID_ARG, "state.n_used is NULL");
  if (reinterpret_cast<uintptr_t>(st->n_used) % 8 != 0)
    return fail(PKM_ERR_INVALID_ARG, "state.n_used must be 8-byte aligned");
  const int64_t rows = int64_t(h->cfg.n_keys) * h->cfg.n_keys2;
  if (st->capacity < 0 || st->capacity > rows)
    return fail(PKM_ERR_INVALID_ARG, "state.capacity must lie in [0, n_keys * n_keys2]");
  PKM_TRY(adam_args(hp, V, st->m, st->v, out));
  out->slot = st->slot;
  out->capacity = st->capacity;
  out->n_used = st->n_used;
  return PKM_OK;
}

// Softmax backward and dq; per-slot sub-key sort keys and coefficients of
// the two halves for the sub-key gradients.
pkm_status run_softmax_bwd(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* idx, const float* w,
                           const float* dw, const void* C, const void* Cp, float* dq, void* ws) {
  const pkm_config& c = h->cfg;
  const BwdLayout L = bwd_layout(h, T);
  // per-slot sort keys and coefficients of the two halves
  uint32_t* key1 = at<uint32_t>(ws, L.key1);
  uint32_t* key2 = at<uint32_t>(ws, L.key2);
  float* coef1 = at<float>(ws, L.ds);
  float* coef2 = at<float>(ws, L.coef2);
  PKM_HIP(launch_softmax_bwd_dq(s, c.dtype, idx, w, dw, C, Cp, T, c.heads, c.d_query, c.topk, c.n_keys, c.n_keys2,
                                1.0f / c.temperature, dq, key1, coef1, key2, coef2),
          "softmax backward / query gradient");
  return PKM_OK;
}

// Sub-key gradients dC, dC' from the per-slot keys and coefficients written by
// run_softmax_bwd.  Touches only its own workspace regions (sort arrays,
// segments, long-run lists), so it may run beside run_query_grad.
pkm_status run_subkey_halves(const pkm_handle_s* h, hipStream_t s, int64_t T, const void* q, float* dC, float* dCp,
                             void* ws) {
  const pkm_config& c = h->cfg;
  const BwdLayout L = bwd_layout(h, T);
  const int64_t N = T * c.heads * c.topk;
  const uint32_t* key1 = at<uint32_t>(ws, L.key1);
  const uint32_t* key2 = at<uint32_t>(ws, L.key2);
  const float* coef1 = at<float>(ws, L.ds);
  const float* coef2 = at<float>(ws, L.coef2);
  for (int half_sel = 0; half_sel < 2; ++half_sel) {
    const int nkeys = half_sel ? c.n_keys2 : c.n_keys;
    float* out = half_sel ? dCp : dC;
    const uint32_t* keys = half_sel ? key2 : key1;
    const float* coef = half_sel ? coef2 : coef1;
    int bits = 1;
    while ((int64_t(1) << bits) <= int64_t(c.heads) * nkeys) ++bits;  // keys <= heads*nkeys (sentinel)
    bool in1 = false;
    PKM_HIP(launch_radix_sort_from(s, keys, at<uint32_t>(ws, L.k0), at<int32_t>(ws, L.v0), at<uint32_t>(ws, L.k1),
                                   at<int32_t>(ws, L.v1), N, bits, at<void>(ws, L.sort_tmp), &in1),
            "sub-key sort");
    const uint32_t* sk = at<uint32_t>(ws, in1 ? L.k1 : L.k0);
    const int32_t* sv = at<int32_t>(ws, in1 ? L.v1 : L.v0);
    int32_t* seg = at<int32_t>(ws, L.seg);
    int64_t* nseg = at<int64_t>(ws, L.nseg) + 1 + half_sel;
    PKM_HIP(launch_fill_f32(s, out, int64_t(c.heads) * nkeys * h->half, 0.f), "sub-key gradient clear");
    PKM_HIP(launch_segments(s, sk, N, seg, nullptr, nseg, at<void>(ws, L.scan_tmp)),
            "sub-key segments");
    PKM_HIP(launch_subkey_grad(s, c.dtype, seg, nseg, int64_t(c.heads) * nkeys, N, sk, sv, coef, q, c.heads,
                               c.d_query, c.topk, half_sel, nkeys, out, at<void>(ws, L.aux)),
            "sub-key gradient");
  }
  return PKM_OK;
}

pkm_status run_subkey_grad(const pkm_handle_s* h, hipStream_t s, int64_t T, const int32_t* idx, const float* w,
                           const float* dw, const void* q, const void* C, const void* Cp, float* dq, float* dC,
                           float* dCp, void* ws) {
  PKM_TRY(run_softmax_bwd(h, s, T, idx, w, dw, C, Cp, dq, ws));
  return run_subkey_halves(h, s, T, q, dC, dCp, ws);
}

pkm_status run_query_grad(const pkm_handle_s* h, hipStream_t s, int64_t T, const float* dq, const void* x,
                          const void* Wq, const float* gamma, const pkm_saved* sv, float* dWq, float* dgamma,
                          float* dbeta, void* dx, void* ws) {
  const pkm_config& c = h->cfg;
  const BwdLayout L = bwd_layout(h, T);
  const bool bn = c.bn == PKM_BN_BATCH;
  if (bn) {
    double* part = at<double>(ws, L.bn_part);
    const int nblk = int((T + kBnRows - 1) / kBnRows);
    PKM_HIP(launch_bn_bwd_partials(s, dq, sv->q_pre, sv->bn_mean, sv->bn_rstd, T, h->F, part),
            "BatchNorm backward partial sums");
    PKM_HIP(launch_bn_bwd_finalize(s, part, nblk, h->F, gamma, dgamma, dbeta, nullptr), "BatchNorm backward finalize");
  }
  void* dqpre = at<void>(ws, L.dqpre);
  void* dqpre_t = at<void>(ws, L.dqpre_t);
  PKM_HIP(launch_bn_bwd_apply(s, c.dtype, dq, sv->q_pre, sv->bn_mean, sv->bn_rstd, gamma, dgamma, dbeta, T, h->F, bn,
                              dqpre, L.ldf, dqpre_t, L.ldt, L.tpad),
          "BatchNorm backward apply");
  // dWq[F, d] = dq_pre^T x : A = dq_pre^T [F, Tpad], B = x^T [d, Tpad]
  void* xt = at<void>(ws, L.x_t);
  PKM_HIP(launch_transpose(s, x, T, c.d_in, c.d_in, xt, L.ldt, L.tpad, h->elem, h->elem), "x transpose");
  float* split = at<float>(ws, L.split);
  const int64_t sstride = int64_t(h->F) * c.d_in;
  if (L.splits == 1) {
    PKM_HIP(launch_gemm_nt(s, c.dtype, h->F, c.d_in, L.tpad, dqpre_t, L.ldt, xt, L.ldt, dWq, c.d_in, false, 1, 0),
            "dWq GEMM");
  } else {
    PKM_HIP(launch_gemm_nt(s, c.dtype, h->F, c.d_in, L.tpad, dqpre_t, L.ldt, xt, L.ldt, split, c.d_in, false,
                           L.splits, sstride),
            "dWq GEMM");
    PKM_HIP(launch_sum_splits(s, split, L.splits, sstride, h->F, c.d_in, c.d_in, dWq, c.d_in, false), "dWq reduce");
  }
  if (dx) {
    // dx[T, d] = dq_pre Wq : A = dq_pre [T, F], B = Wq^T [d, F]
    void* wqt = at<void>(ws, L.wq_t);
    PKM_HIP(launch_transpose(s, Wq, h->F, c.d_in, c.d_in, wqt, L.ldf, h->F, h->elem, h->elem), "Wq transpose");
    PKM_HIP(launch_gemm_nt(s, c.dtype, T, c.d_in, h->F, dqpre, L.ldf, wqt, L.ldf, dx, c.d_in, c.dtype == PKM_BF16, 1, 0),
            "dx GEMM");
  }
  return PKM_OK;
}

pkm_status check_saved(const pkm_handle_s* h, const pkm_saved* sv, bool need_sel) {
  if (sv == nullptr) return fail(PKM_ERR_INVALID_ARG, "saved is NULL");
  if (need_sel) {
    PKM_TRY(need(sv->idx, "saved->idx"));
    PKM_TRY(need(sv->w, "saved->w"));
  }
  PKM_TRY(need(sv->q, "saved->q"));
  PKM_TRY(need(sv->q_pre, "saved->q_pre"));
  if (h->cfg.bn == PKM_BN_BATCH) {
    PKM_TRY(need(sv->bn_mean, "saved->bn_mean"));
    PKM_TRY(need(sv->bn_rstd, "saved->bn_rstd"));
  }
  return PKM_OK;
}

pkm_status zero_grads(const pkm_handle_s* h, hipStream_t s, int64_t* n_touched, float* dC, float* dCp, float* dWq,
                      float* dgamma, float* dbeta) {
  const pkm_config& c = h->cfg;
  // a fill kernel rather than a memset node (safe under stream capture)
  if (n_touched) PKM_HIP(launch_fill_f32(s, reinterpret_cast<float*>(n_touched), 2, 0.f), "clear n_touched");
  if (dC) PKM_HIP(launch_fill_f32(s, dC, int64_t(c.heads) * c.n_keys * h->half, 0.f), "clear dC");
  if (dCp) PKM_HIP(launch_fill_f32(s, dCp, int64_t(c.heads) * c.n_keys2 * h->half, 0.f), "clear dCp");
  if (dWq) PKM_HIP(launch_fill_f32(s, dWq, int64_t(h->F) * c.d_in, 0.f), "clear dWq");
  if (dgamma) PKM_HIP(launch_fill_f32(s, dgamma, h->F, 0.f), "clear dgamma");
  if (dbeta) PKM_HIP(launch_fill_f32(s, dbeta, h->F, 0.f), "clear dbeta");
  return PKM_OK;
}

// pkm_forward's argument checks (everything but the workspace), before any HIP call.
pkm_status check_forward_args(pkm_handle_t handle, int64_t T, const void* x, const void* Wq, const float* bn_gamma,
                              const float* bn_beta, const void* C, const void* Cp, const void* V, const void* y,
                              const pkm_saved* saved) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(x, "x"));
  PKM_TRY(need(Wq, "Wq"));
  PKM_TRY(need(C, "C"));
  PKM_TRY(need(Cp, "Cp"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(y, "y"));
  if (handle->cfg.bn == PKM_BN_BATCH) {
    PKM_TRY(need(bn_gamma, "bn_gamma"));
    PKM_TRY(need(bn_beta, "bn_beta"));
  }
  return check_saved(handle, saved, true);
}

}  // namespace

// ---- pkm_forward_noalloc: the forward with its workspace in a static device array ----
//
// For callers that cannot allocate (code under graph capture, tight serving
// loops): the forward's workspace regions (per-half lists, BatchNorm partial
// sums, packed sub-keys) live in `scratch`, one copy per device, held until
// the process ends.  Every region is written before it is read within a call,
// so nothing needs clearing.  Calls on one device share the array: calls that
// overlap in time on one device (different streams, or host threads without
// ordering) race.
constexpr size_t kNoAllocScratchBytes = size_t(128) << 20;
constexpr int kNoAllocMaxDevices = 64;

static __device__ __attribute__((aligned(256))) unsigned char scratch[kNoAllocScratchBytes];

namespace {

std::mutex g_scratch_mu;
void* g_scratch_ptr[kNoAllocMaxDevices];  // device address of `scratch` per device, null until first use

// The device address of the current device's copy of `scratch` (looked up
// once per device, with that device current; the name itself is only a host
// stand-in and must never reach a kernel).
pkm_status scratch_for_current_device(void** out) {
  int dev = -1;
  PKM_HIP(hipGetDevice(&dev), "hipGetDevice");
  if (dev < 0 || dev >= kNoAllocMaxDevices)
    return fail(PKM_ERR_UNSUPPORTED, "device %d is beyond the %d devices pkm_forward_noalloc serves", dev,
                kNoAllocMaxDevices);
  std::lock_guard<std::mutex> lock(g_scratch_mu);
  if (g_scratch_ptr[dev] == nullptr) {
    void* p = nullptr;
    PKM_HIP(hipGetSymbolAddress(&p, HIP_SYMBOL(scratch)), "hipGetSymbolAddress(scratch)");
    if (p == nullptr || !aligned16(p)) return fail(PKM_ERR_HIP, "scratch has no usable device address");
    g_scratch_ptr[dev] = p;
  }
  *out = g_scratch_ptr[dev];
  return PKM_OK;
}

}  // namespace

extern "C" {

const char* pkm_status_string(pkm_status s) {
  switch (s) {
    case PKM_OK: return "ok";
    case PKM_ERR_INVALID_ARG: return "invalid argument";
    case PKM_ERR_UNSUPPORTED: return "unsupported configuration";
    case PKM_ERR_WORKSPACE: return "workspace missing or too small";
    case PKM_ERR_HIP: return "HIP error";
  }
  return "unknown status";
}

const char* pkm_last_error(void) { return g_err.c_str(); }

pkm_status pkm_create(const pkm_config* cfg, pkm_handle_t* out) {
  if (cfg == nullptr || out == nullptr) return fail(PKM_ERR_INVALID_ARG, "cfg or out is NULL");
  *out = nullptr;
  const pkm_config& c = *cfg;
  if (c.dtype != PKM_F32 && c.dtype != PKM_BF16) return fail(PKM_ERR_INVALID_ARG, "dtype %d unknown", c.dtype);
  if (c.bn != PKM_BN_NONE && c.bn != PKM_BN_BATCH) return fail(PKM_ERR_INVALID_ARG, "bn mode %d unknown", c.bn);
  const int vec = c.dtype == PKM_BF16 ? 8 : 4;  // elements per 16 bytes
  if (c.d_in < 1) return fail(PKM_ERR_INVALID_ARG, "d_in = %d < 1", c.d_in);
  if (c.heads < 1) return fail(PKM_ERR_INVALID_ARG, "heads = %d < 1", c.heads);
  if (c.d_query < 2 || c.d_query % 2) return fail(PKM_ERR_INVALID_ARG, "d_query = %d must be even and >= 2", c.d_query);
  if (c.n_keys < 1 || c.n_keys2 < 1) return fail(PKM_ERR_INVALID_ARG, "n_keys and n_keys2 must be >= 1");
  if (c.topk < 1) return fail(PKM_ERR_INVALID_ARG, "topk = %d < 1", c.topk);
  if (c.topk > c.n_keys || c.topk > c.n_keys2)
    return fail(PKM_ERR_INVALID_ARG, "topk = %d exceeds a codebook size (%d, %d)", c.topk, c.n_keys, c.n_keys2);
  if (c.d_value < 1) return fail(PKM_ERR_INVALID_ARG, "d_value = %d < 1", c.d_value);
  if (!(c.temperature > 0.0f)) return fail(PKM_ERR_INVALID_ARG, "temperature must be > 0");
  if (c.bn == PKM_BN_BATCH && !(c.bn_eps >= 0.0f)) return fail(PKM_ERR_INVALID_ARG, "bn_eps must be >= 0");
  if (int64_t(c.n_keys) * c.n_keys2 >= (int64_t(1) << 31))
    return fail(PKM_ERR_INVALID_ARG, "n_keys * n_keys2 = %lld does not fit int32 row ids",
                (long long)(int64_t(c.n_keys) * c.n_keys2));
  // limits of the kernels
  if (c.topk > 32) return fail(PKM_ERR_UNSUPPORTED, "topk = %d > 32", c.topk);
  if (c.n_keys > 2048 || c.n_keys2 > 2048) return fail(PKM_ERR_UNSUPPORTED, "codebooks larger than 2048 sub-keys");
  if (c.d_in % vec) return fail(PKM_ERR_UNSUPPORTED, "d_in must be a multiple of %d for this dtype", vec);
  if ((c.d_query / 2) % vec)
    return fail(PKM_ERR_UNSUPPORTED, "d_query/2 must be a multiple of %d for this dtype", vec);
  if (c.d_value % vec) return fail(PKM_ERR_UNSUPPORTED, "d_value must be a multiple of %d for this dtype", vec);
  if (c.d_value / vec > 256)
    return fail(PKM_ERR_UNSUPPORTED, "d_value rows above 4096 bytes are not supported");
  if (c.value_format != PKM_VALUES_STORAGE && c.value_format != PKM_VALUES_FP8)
    return fail(PKM_ERR_INVALID_ARG, "value_format %d unknown", c.value_format);
  if (c.score_fn != PKM_SCORE_DOT && c.score_fn != PKM_SCORE_IDW)
    return fail(PKM_ERR_INVALID_ARG, "score_fn %d unknown", c.score_fn);
  if (c.value_format == PKM_VALUES_FP8 && c.d_value % 16)
    return fail(PKM_ERR_UNSUPPORTED, "fp8 values need d_value to be a multiple of 16");
  const int maxk = c.n_keys > c.n_keys2 ? c.n_keys : c.n_keys2;
  if (!score_topk_supported(c.dtype, c.d_query / 2, maxk))
    return fail(PKM_ERR_UNSUPPORTED, "d_query/2 = %d with %d sub-keys does not fit the scoring tile", c.d_query / 2,
                maxk);
  pkm_handle_s* h = new (std::nothrow) pkm_handle_s;
  if (!h) return fail(PKM_ERR_INVALID_ARG, "out of host memory");
  h->cfg = c;
  h->half = c.d_query / 2;
  h->F = c.heads * c.d_query;
  h->elem = c.dtype == PKM_BF16 ? 2 : 4;
  int bits = 0;
  while ((int64_t(1) << bits) < int64_t(c.n_keys) * c.n_keys2) ++bits;
  h->row_bits = bits;
  // side stream on the current device (default priority); without a device the
  // backward simply stays on the caller's stream
  h->device = -1;
  h->cus = 256;
  h->side = nullptr;
  h->fork = h->join = nullptr;
  int dev = -1;
  if (hipGetDevice(&dev) == hipSuccess) {
    int cus = 0;
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) == hipSuccess && cus > 0)
      h->cus = cus;
    hipStream_t st = nullptr;
    hipEvent_t e1 = nullptr, e2 = nullptr;
    if (hipStreamCreateWithFlags(&st, hipStreamNonBlocking) == hipSuccess &&
        hipEventCreateWithFlags(&e1, hipEventDisableTiming) == hipSuccess &&
        hipEventCreateWithFlags(&e2, hipEventDisableTiming) == hipSuccess) {
      h->device = dev;
      h->side = st;
      h->fork = e1;
      h->join = e2;
    } else {
      if (st) (void)hipStreamDestroy(st);
      if (e1) (void)hipEventDestroy(e1);
      if (e2) (void)hipEventDestroy(e2);
    }
  }
  (void)hipGetLastError();  // a failed creation above must not surface in a later call's status
  *out = h;
  return PKM_OK;
}

pkm_status pkm_destroy(pkm_handle_t handle) {
  if (handle != nullptr && handle->side != nullptr) {
    int prev = -1;
    const bool switched = hipGetDevice(&prev) == hipSuccess && prev != handle->device &&
                          hipSetDevice(handle->device) == hipSuccess;
    (void)hipStreamDestroy(handle->side);
    (void)hipEventDestroy(handle->fork);
    (void)hipEventDestroy(handle->join);
    if (switched) (void)hipSetDevice(prev);
  }
  delete handle;
  return PKM_OK;
}

pkm_status pkm_get_config(pkm_handle_t handle, pkm_config* out) {
  PKM_TRY(check_handle(handle));
  if (!out) return fail(PKM_ERR_INVALID_ARG, "out is NULL");
  *out = handle->cfg;
  return PKM_OK;
}

pkm_status pkm_workspace_size(pkm_handle_t handle, int64_t T, int with_backward, size_t* bytes) {
  PKM_TRY(check_handle(handle));
  if (!bytes) return fail(PKM_ERR_INVALID_ARG, "bytes is NULL");
  PKM_TRY(check_T(handle, T));
  if (with_backward != PKM_WS_FORWARD && with_backward != PKM_WS_BACKWARD && with_backward != PKM_WS_FWPKM_CHUNK)
    return fail(PKM_ERR_INVALID_ARG, "with_backward = %d is none of 0, 1, 2", with_backward);
  *bytes = ws_size(handle, T, with_backward);
  return PKM_OK;
}

pkm_status pkm_forward(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                       const float* bn_gamma, const float* bn_beta, const void* C, const void* Cp, const void* V,
                       void* y, const pkm_saved* saved, void* ws, size_t ws_bytes) {
  PKM_TRY(check_forward_args(handle, T, x, Wq, bn_gamma, bn_beta, C, Cp, V, y, saved));
  PKM_TRY(check_ws(handle, T, 0, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  hipStream_t s = as_stream(stream);
  const FwdLayout L = fwd_layout(handle, T);
  int32_t* sub_idx = at<int32_t>(ws, L.sub_idx);
  float* sub_score = at<float>(ws, L.sub_score);
  PKM_TRY(run_query(handle, s, T, x, Wq, bn_gamma, bn_beta, saved, ws));
  PKM_TRY(run_score(handle, s, T, saved->q, C, Cp, sub_idx, sub_score, ws));
  const pkm_config& c = handle->cfg;
  const bool fp8 = c.value_format == PKM_VALUES_FP8;
  if (merge_gather_supported(c.dtype, c.topk, c.d_value, fp8)) {
    PKM_HIP(launch_merge_gather(s, c.dtype, sub_idx, sub_score, T, c.heads, c.topk, c.n_keys2, 1.0f / c.temperature,
                                saved->idx, saved->w, V, y, c.d_value, fp8),
            "candidate merge / softmax + value gather-sum");
    return PKM_OK;
  }
  PKM_TRY(run_merge(handle, s, T, sub_idx, sub_score, saved->idx, saved->w, nullptr));
  PKM_TRY(run_gather(handle, s, T, saved->idx, saved->w, V, y));
  return PKM_OK;
}

pkm_status pkm_forward_noalloc(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                               const float* bn_gamma, const float* bn_beta, const void* C, const void* Cp,
                               const void* V, void* y, const pkm_saved* saved) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  const size_t want = ws_size(handle, T, PKM_WS_FORWARD);
  if (want > kNoAllocScratchBytes)
    return fail(PKM_ERR_WORKSPACE,
                "pkm_forward_noalloc: T = %lld needs %zu bytes of workspace, above its static %zu-byte scratch; "
                "use pkm_forward with a caller workspace",
                (long long)T, want, kNoAllocScratchBytes);
  PKM_TRY(check_forward_args(handle, T, x, Wq, bn_gamma, bn_beta, C, Cp, V, y, saved));
  void* ws = nullptr;
  PKM_TRY(scratch_for_current_device(&ws));
  return pkm_forward(handle, stream, T, x, Wq, bn_gamma, bn_beta, C, Cp, V, y, saved, ws, kNoAllocScratchBytes);
}

// pkm_backward (adam == null: dV written) and pkm_backward_adam (Adam step on
// the touched rows of V instead of dV).
static pkm_status backward_impl(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                                const void* Wq, const float* bn_gamma, const void* C, const void* Cp, const void* V,
                                const pkm_saved* saved, float* dV, const VgAdam* adam, int32_t* touched,
                                int64_t* n_touched, float* dC, float* dCp, float* dWq, float* dgamma, float* dbeta,
                                void* dx, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(need_dot_scores(handle));
  PKM_TRY(check_T(handle, T));
  const bool bn = handle->cfg.bn == PKM_BN_BATCH;
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(x, "x"));
  PKM_TRY(need(Wq, "Wq"));
  PKM_TRY(need(C, "C"));
  PKM_TRY(need(Cp, "Cp"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(check_saved(handle, saved, true));
  if (adam == nullptr) PKM_TRY(need(dV, "dV"));
  PKM_TRY(need(touched, "touched"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(need(dC, "dC"));
  PKM_TRY(need(dCp, "dCp"));
  PKM_TRY(need(dWq, "dWq"));
  if (bn) {
    PKM_TRY(need(bn_gamma, "bn_gamma"));
    PKM_TRY(need(dgamma, "dgamma"));
    PKM_TRY(need(dbeta, "dbeta"));
  }
  if (dx) PKM_TRY(need(dx, "dx"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, n_touched, dC, dCp, dWq, bn ? dgamma : nullptr, bn ? dbeta : nullptr);
  const BwdLayout L = bwd_layout(handle, T);
  float* dw = at<float>(ws, L.dw);
  float* dq = at<float>(ws, L.dq);
  PKM_TRY(run_value_grad(handle, s, T, saved->idx, saved->w, dY, V, dV, touched, n_touched, dw, ws, adam));
  PKM_TRY(run_softmax_bwd(handle, s, T, saved->idx, saved->w, dw, C, Cp, dq, ws));
  // The sub-key gradients (sorts, L2 gathers) and the projection gradients
  // (BatchNorm backward, MFMA GEMMs) only share inputs: run them side by side.
  int dev = -1;
  pkm_handle_s* hm = const_cast<pkm_handle_s*>(handle);
  if (hm->side != nullptr && hipGetDevice(&dev) == hipSuccess && dev == hm->device) {
    std::lock_guard<std::mutex> lock(hm->side_mu);
    PKM_HIP(hipEventRecord(hm->fork, s), "fork event");
    PKM_HIP(hipStreamWaitEvent(hm->side, hm->fork, 0), "side stream wait");
    const pkm_status side_st = run_subkey_halves(handle, hm->side, T, saved->q, dC, dCp, ws);
    const hipError_t joined = hipEventRecord(hm->join, hm->side);
    const pkm_status main_st = run_query_grad(handle, s, T, dq, x, Wq, bn_gamma, saved, dWq,
                                              bn ? dgamma : nullptr, bn ? dbeta : nullptr, dx, ws);
    // the caller's stream waits for the side stream whatever failed above, so
    // that no work queued there outlives the call unordered
    const hipError_t waited =
        joined == hipSuccess ? hipStreamWaitEvent(s, hm->join, 0) : hipStreamSynchronize(hm->side);
    PKM_TRY(side_st);
    PKM_TRY(main_st);
    PKM_HIP(joined, "join event");
    PKM_HIP(waited, "join wait");
    return PKM_OK;
  }
  PKM_TRY(run_subkey_halves(handle, s, T, saved->q, dC, dCp, ws));
  PKM_TRY(run_query_grad(handle, s, T, dq, x, Wq, bn_gamma, saved, dWq, bn ? dgamma : nullptr, bn ? dbeta : nullptr,
                         dx, ws));
  return PKM_OK;
}

pkm_status pkm_backward(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x, const void* Wq,
                        const float* bn_gamma, const void* C, const void* Cp, const void* V, const pkm_saved* saved,
                        float* dV, int32_t* touched, int64_t* n_touched, float* dC, float* dCp, float* dWq,
                        float* dgamma, float* dbeta, void* dx, void* ws, size_t ws_bytes) {
  return backward_impl(handle, stream, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, dV, nullptr, touched, n_touched, dC,
                       dCp, dWq, dgamma, dbeta, dx, ws, ws_bytes);
}

pkm_status pkm_backward_adam(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                             const void* Wq, const float* bn_gamma, const void* C, const void* Cp, void* V,
                             const pkm_saved* saved, float* adam_m, float* adam_v, const pkm_adam* adam,
                             int32_t* touched, int64_t* n_touched, float* dC, float* dCp, float* dWq, float* dgamma,
                             float* dbeta, void* dx, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(adam_m, "adam_m"));
  PKM_TRY(need(adam_v, "adam_v"));
  VgAdam ad;
  PKM_TRY(adam_args(adam, V, adam_m, adam_v, &ad));
  return backward_impl(handle, stream, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, nullptr, &ad, touched, n_touched, dC,
                       dCp, dWq, dgamma, dbeta, dx, ws, ws_bytes);
}

pkm_status pkm_backward_adam_rows(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                                  const void* Wq, const float* bn_gamma, const void* C, const void* Cp, void* V,
                                  const pkm_saved* saved, const pkm_adam_rows* state, const pkm_adam* adam,
                                  int32_t* touched, int64_t* n_touched, float* dC, float* dCp, float* dWq,
                                  float* dgamma, float* dbeta, void* dx, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need(V, "V"));
  VgAdam ad;
  PKM_TRY(adam_rows_args(handle, adam, V, state, &ad));
  return backward_impl(handle, stream, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, nullptr, &ad, touched, n_touched, dC,
                       dCp, dWq, dgamma, dbeta, dx, ws, ws_bytes);
}

pkm_status pkm_stage_query(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                           const float* bn_gamma, const float* bn_beta, const pkm_saved* saved, void* ws,
                           size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(x, "x"));
  PKM_TRY(need(Wq, "Wq"));
  if (handle->cfg.bn == PKM_BN_BATCH) {
    PKM_TRY(need(bn_gamma, "bn_gamma"));
    PKM_TRY(need(bn_beta, "bn_beta"));
  }
  PKM_TRY(check_saved(handle, saved, false));
  PKM_TRY(check_ws(handle, T, 0, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  return run_query(handle, as_stream(stream), T, x, Wq, bn_gamma, bn_beta, saved, ws);
}

pkm_status pkm_stage_score_topk(pkm_handle_t handle, void* stream, int64_t T, const void* q, const void* C,
                                const void* Cp, int32_t* sub_idx, float* sub_score, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(q, "q"));
  PKM_TRY(need(C, "C"));
  PKM_TRY(need(Cp, "Cp"));
  PKM_TRY(need(sub_idx, "sub_idx"));
  PKM_TRY(need(sub_score, "sub_score"));
  PKM_TRY(check_ws(handle, T, 0, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  return run_score(handle, as_stream(stream), T, q, C, Cp, sub_idx, sub_score, ws);
}

pkm_status pkm_stage_merge_softmax(pkm_handle_t handle, void* stream, int64_t T, const int32_t* sub_idx,
                                   const float* sub_score, int32_t* idx, float* w, float* score) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(sub_idx, "sub_idx"));
  PKM_TRY(need(sub_score, "sub_score"));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  if (score) PKM_TRY(need(score, "score"));
  if (T == 0) return PKM_OK;
  return run_merge(handle, as_stream(stream), T, sub_idx, sub_score, idx, w, score);
}

pkm_status pkm_stage_gather(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                            const void* V, void* y) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(y, "y"));
  if (T == 0) return PKM_OK;
  return run_gather(handle, as_stream(stream), T, idx, w, V, y);
}

pkm_status pkm_stage_value_grad(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                                const void* dY, const void* V, float* dV, int32_t* touched, int64_t* n_touched,
                                float* dw, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(dV, "dV"));
  PKM_TRY(need(touched, "touched"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(need(dw, "dw"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, n_touched, nullptr, nullptr, nullptr, nullptr, nullptr);
  return run_value_grad(handle, s, T, idx, w, dY, V, dV, touched, n_touched, dw, ws);
}

pkm_status pkm_stage_value_adam(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                                const void* dY, void* V, float* adam_m, float* adam_v, const pkm_adam* adam,
                                int32_t* touched, int64_t* n_touched, float* dw, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(adam_m, "adam_m"));
  PKM_TRY(need(adam_v, "adam_v"));
  VgAdam ad;
  PKM_TRY(adam_args(adam, V, adam_m, adam_v, &ad));
  PKM_TRY(need(touched, "touched"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(need(dw, "dw"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, n_touched, nullptr, nullptr, nullptr, nullptr, nullptr);
  return run_value_grad(handle, s, T, idx, w, dY, V, nullptr, touched, n_touched, dw, ws, &ad);
}

pkm_status pkm_stage_value_adam_rows(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                     const float* w, const void* dY, void* V, const pkm_adam_rows* state,
                                     const pkm_adam* adam, int32_t* touched, int64_t* n_touched, float* dw,
                                     void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(V, "V"));
  VgAdam ad;
  PKM_TRY(adam_rows_args(handle, adam, V, state, &ad));
  PKM_TRY(need(touched, "touched"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(need(dw, "dw"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, n_touched, nullptr, nullptr, nullptr, nullptr, nullptr);
  return run_value_grad(handle, s, T, idx, w, dY, V, nullptr, touched, n_touched, dw, ws, &ad);
}

pkm_status pkm_diagnostics(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                           int32_t* hits_c, int32_t* hits_cp, int64_t* used, float* entropy, double* entropy_sum,
                           void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(hits_c, "hits_c"));
  PKM_TRY(need(hits_cp, "hits_cp"));
  if (used == nullptr) return fail(PKM_ERR_INVALID_ARG, "used is NULL");
  if (reinterpret_cast<uintptr_t>(used) % 8 != 0) return fail(PKM_ERR_INVALID_ARG, "used is not 8-byte aligned");
  if (entropy) PKM_TRY(need(entropy, "entropy"));
  if (entropy_sum && reinterpret_cast<uintptr_t>(entropy_sum) % 8 != 0)
    return fail(PKM_ERR_INVALID_ARG, "entropy_sum is not 8-byte aligned");
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  const pkm_config& c = handle->cfg;
  PKM_HIP(launch_diagnostics(as_stream(stream), idx, w, T, c.heads, c.topk, c.n_keys, c.n_keys2, hits_c, hits_cp,
                             used, entropy, entropy_sum, ws),
          "diagnostics");
  return PKM_OK;
}

pkm_status pkm_quantize_values(pkm_handle_t handle, void* stream, const void* V_src, int64_t rows, void* V_fp8) {
  PKM_TRY(check_handle(handle));
  const pkm_config& c = handle->cfg;
  if (c.value_format != PKM_VALUES_FP8)
    return fail(PKM_ERR_INVALID_ARG, "pkm_quantize_values needs a handle with value_format = PKM_VALUES_FP8");
  if (rows < 0) return fail(PKM_ERR_INVALID_ARG, "rows = %lld < 0", (long long)rows);
  if (rows > int64_t(c.n_keys) * c.n_keys2)
    return fail(PKM_ERR_INVALID_ARG, "rows = %lld exceeds the table (%lld rows)", (long long)rows,
                (long long)(int64_t(c.n_keys) * c.n_keys2));
  PKM_TRY(need(V_src, "V_src"));
  PKM_TRY(need(V_fp8, "V_fp8"));
  if (rows == 0) return PKM_OK;
  PKM_HIP(launch_quantize_fp8(as_stream(stream), c.dtype, V_src, rows, c.d_value, V_fp8), "fp8 value quantization");
  return PKM_OK;
}

pkm_status pkm_stage_row_groups(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, int32_t* touched,
                                int64_t* n_touched, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(touched, "touched"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, n_touched, nullptr, nullptr, nullptr, nullptr, nullptr);
  return run_row_groups(handle, s, T, idx, touched, n_touched, ws);
}

pkm_status pkm_stage_value_grad_grouped(pkm_handle_t handle, void* stream, int64_t T, const float* w, const void* dY,
                                        const void* V, float* dV, float* dw, const int64_t* n_touched, void* ws,
                                        size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(dV, "dV"));
  PKM_TRY(need(dw, "dw"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  return run_value_grad_grouped(handle, as_stream(stream), T, w, dY, V, dV, dw, n_touched, ws);
}

pkm_status pkm_stage_value_adam_grouped(pkm_handle_t handle, void* stream, int64_t T, const float* w, const void* dY,
                                        void* V, float* adam_m, float* adam_v, const pkm_adam* adam, float* dw,
                                        const int64_t* n_touched, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dY, "dY"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(adam_m, "adam_m"));
  PKM_TRY(need(adam_v, "adam_v"));
  VgAdam ad;
  PKM_TRY(adam_args(adam, V, adam_m, adam_v, &ad));
  PKM_TRY(need(dw, "dw"));
  if (n_touched == nullptr) return fail(PKM_ERR_INVALID_ARG, "n_touched is NULL");
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  return run_value_grad_grouped(handle, as_stream(stream), T, w, dY, V, nullptr, dw, n_touched, ws, &ad);
}

pkm_status pkm_stage_subkey_grad(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                                 const float* dw, const void* q, const void* C, const void* Cp, float* dq, float* dC,
                                 float* dCp, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_dot_scores(handle));
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  PKM_TRY(need(dw, "dw"));
  PKM_TRY(need(q, "q"));
  PKM_TRY(need(C, "C"));
  PKM_TRY(need(Cp, "Cp"));
  PKM_TRY(need(dq, "dq"));
  PKM_TRY(need(dC, "dC"));
  PKM_TRY(need(dCp, "dCp"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, nullptr, dC, dCp, nullptr, nullptr, nullptr);
  return run_subkey_grad(handle, s, T, idx, w, dw, q, C, Cp, dq, dC, dCp, ws);
}

pkm_status pkm_stage_query_grad(pkm_handle_t handle, void* stream, int64_t T, const float* dq, const void* x,
                                const void* Wq, const float* bn_gamma, const pkm_saved* saved, float* dWq,
                                float* dgamma, float* dbeta, void* dx, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(check_T(handle, T));
  const bool bn = handle->cfg.bn == PKM_BN_BATCH;
  PKM_TRY(need(dq, "dq"));
  PKM_TRY(need(x, "x"));
  PKM_TRY(need(Wq, "Wq"));
  PKM_TRY(check_saved(handle, saved, false));
  PKM_TRY(need(dWq, "dWq"));
  if (bn) {
    PKM_TRY(need(bn_gamma, "bn_gamma"));
    PKM_TRY(need(dgamma, "dgamma"));
    PKM_TRY(need(dbeta, "dbeta"));
  }
  if (dx) PKM_TRY(need(dx, "dx"));
  PKM_TRY(check_ws(handle, T, 1, ws, ws_bytes));
  hipStream_t s = as_stream(stream);
  if (T == 0) return zero_grads(handle, s, nullptr, nullptr, nullptr, dWq, bn ? dgamma : nullptr, bn ? dbeta : nullptr);
  return run_query_grad(handle, s, T, dq, x, Wq, bn_gamma, saved, dWq, bn ? dgamma : nullptr, bn ? dbeta : nullptr,
                        dx, ws);
}

}  // extern "C"

namespace {

// pkm_fwpkm_chunk over consecutive slices of call_T tokens, in order.  The
// selection reads only q, C and C', never V, so it runs once over all T tokens
// (the merge's table offsets cycle over the streams every call_T tokens); then
// each slice runs its gather with the residual and its value step.
pkm_status fwpkm_calls(pkm_handle_t handle, void* stream, int64_t T, int64_t call_T, int64_t streams,
                       const void* q, const void* C, const void* Cp, void* V, const void* target, float lr, void* y,
                       int32_t* idx, float* w, void* ws, size_t ws_bytes) {
  PKM_TRY(check_handle(handle));
  PKM_TRY(need_storage_values(handle));
  if (handle->cfg.score_fn != PKM_SCORE_IDW)
    return fail(PKM_ERR_UNSUPPORTED, "the memorization chunk scores with score_fn = PKM_SCORE_IDW");
  PKM_TRY(check_T(handle, T));
  PKM_TRY(need(q, "q"));
  PKM_TRY(need(C, "C"));
  PKM_TRY(need(Cp, "Cp"));
  PKM_TRY(need(V, "V"));
  PKM_TRY(need(target, "target"));
  PKM_TRY(need(y, "y"));
  PKM_TRY(need(idx, "idx"));
  PKM_TRY(need(w, "w"));
  if (!(std::isfinite(lr) && lr >= 0.f)) return fail(PKM_ERR_INVALID_ARG, "lr must be finite and >= 0");
  if (streams < 1) return fail(PKM_ERR_INVALID_ARG, "streams = %lld < 1", (long long)streams);
  if (call_T < 1 || T % call_T)
    return fail(PKM_ERR_INVALID_ARG, "T = %lld is not a multiple of call_T = %lld", (long long)T, (long long)call_T);
  if (call_T % streams)
    return fail(PKM_ERR_INVALID_ARG, "call_T = %lld is not a multiple of streams = %lld", (long long)call_T,
                (long long)streams);
  const pkm_config& c = handle->cfg;
  const int64_t rows = streams * int64_t(c.n_keys) * c.n_keys2;
  if (rows >= (int64_t(1) << 31))
    return fail(PKM_ERR_UNSUPPORTED, "streams * |C| * |C'| = %lld does not fit int32 row ids", (long long)rows);
  PKM_TRY(check_ws(handle, T, PKM_WS_FWPKM_CHUNK, ws, ws_bytes));
  if (T == 0) return PKM_OK;
  int bits = 0;
  while ((int64_t(1) << bits) < rows) ++bits;
  hipStream_t s = as_stream(stream);
  const FwdLayout F = fwd_layout(handle, T);
  const ChunkLayout L = chunk_layout(handle, T);
  int32_t* sub_idx = at<int32_t>(ws, F.sub_idx);
  float* sub_score = at<float>(ws, F.sub_score);
  PKM_TRY(run_score(handle, s, T, q, C, Cp, sub_idx, sub_score, ws));
  const int64_t R = int64_t(c.heads) * c.topk;
  const size_t row_bytes = size_t(c.d_value) * size_t(handle->elem);
  const int64_t calls = T / call_T, n_call = call_T * R;
  // one call of one stream: the merge, the gather and the residual in one launch
  const bool fused = streams == 1 && calls == 1 && merge_gather_supported(c.dtype, c.topk, c.d_value, false);
  if (!fused)
    PKM_TRY(run_merge(handle, s, T, sub_idx, sub_score, idx, w, nullptr, streams > 1 ? call_T / streams : 0, streams));
  // the slices' steps reuse the scoring's workspace (its results are in idx and w)
  if (streams == 1 && calls > 1 && calls <= kSortGroupsMax && n_call <= kSmallSortMax) {
    // One stream whose calls each fit one workgroup's grouping: every call's
    // grouping (and long-run plan) in one launch of a workgroup per call, up
    // front (it reads only idx), then per call the gather with the residual
    // and the value step on that call's own table of row segments.  Lookup ids,
    // segment positions and the residual rows are global, so the per-row sums
    // run over the same lookups in the same order as in separate calls.
    const BwdLayout B = bwd_layout(handle, T);
    uint32_t* sk = at<uint32_t>(ws, B.k0);
    int32_t* sv = at<int32_t>(ws, B.v0);
    int32_t* seg_g = at<int32_t>(ws, B.grp);                                            // calls x (n_call + 1)
    int64_t* cnt_g = reinterpret_cast<int64_t*>(seg_g + 2 * T * R + kSortGroupsMax);  // calls
    void* plans = at<void>(ws, L.plans);
    PKM_HIP(launch_sort_segments_separate(s, reinterpret_cast<const uint32_t*>(idx), T * R, int(calls), bits, sk, sv,
                                          seg_g, cnt_g, plans),
            "row grouping of every call");
    char* e = at<char>(ws, L.e);  // T rows: residual rows sit at their tokens' positions
    VgAdam sgd{};
    sgd.V = V;
    sgd.step_size = lr;
    sgd.sgd = 1;
    for (int64_t g = 0; g < calls; ++g) {
      const int64_t t0 = g * call_T;
      PKM_HIP(launch_gather(s, c.dtype, idx + t0 * R, w + t0 * R, V, static_cast<char*>(y) + t0 * row_bytes, call_T,
                            int(R), c.d_value, false, static_cast<const char*>(target) + t0 * row_bytes,
                            e + t0 * row_bytes),
              "value gather-sum and reconstruction residual");
      const VgPlan plan = group_plan(plans, int(g));
      PKM_HIP(launch_value_grad(s, c.dtype, seg_g + g * (n_call + 1), cnt_g + g, n_call, sk, sv, w, e, V, nullptr,
                                at<float>(ws, B.dw), int(R), c.d_value, c.accumulate_dv != 0, at<void>(ws, B.aux),
                                &sgd, true, &plan),
              "value step");
    }
    return PKM_OK;
  }
  const int64_t n_grp = streams > 0 ? n_call / streams : 0;
  if (streams > 1 && calls > 1 && calls * streams <= kSortGroupsMax && n_grp <= kSmallSortMax) {
    // A batch of streams: every (call, stream) chunk grouped up front by its
    // own workgroup; per call the gather with the residual, one join of that
    // call's streams' tables (their rows lie in separate tables, so the
    // tables side by side are the call's sorted whole) with its long-run plan,
    // and the value step.  Same lookups in the same order per row as separate
    // calls.
    const BwdLayout B = bwd_layout(handle, T);
    uint32_t* sk = at<uint32_t>(ws, B.k0);
    int32_t* sv = at<int32_t>(ws, B.v0);
    int32_t* seg_g = at<int32_t>(ws, B.grp);
    int64_t* cnt_g = reinterpret_cast<int64_t*>(seg_g + 2 * T * R + kSortGroupsMax);
    PKM_HIP(launch_sort_segments_separate(s, reinterpret_cast<const uint32_t*>(idx), T * R, int(calls * streams),
                                          bits, sk, sv, seg_g, cnt_g, at<void>(ws, L.plans)),
            "row grouping of every call and stream");
    char* e = at<char>(ws, L.e);
    int32_t* seg = at<int32_t>(ws, B.seg);
    int64_t* nseg = at<int64_t>(ws, L.n_touched);
    const VgPlan plan = value_grad_plan(at<void>(ws, B.aux), n_call, c.d_value);
    VgAdam sgd{};
    sgd.V = V;
    sgd.step_size = lr;
    sgd.sgd = 1;
    for (int64_t g = 0; g < calls; ++g) {
      const int64_t t0 = g * call_T;
      PKM_HIP(launch_gather(s, c.dtype, idx + t0 * R, w + t0 * R, V, static_cast<char*>(y) + t0 * row_bytes, call_T,
                            int(R), c.d_value, false, static_cast<const char*>(target) + t0 * row_bytes,
                            e + t0 * row_bytes),
              "value gather-sum and reconstruction residual");
      PKM_HIP(launch_join_groups(s, seg_g + g * streams * (n_grp + 1), cnt_g + g * streams, int(streams), int(n_grp),
                                 (g + 1) * n_call, seg, nseg, &plan),
              "row segments of the call");
      PKM_HIP(launch_value_grad(s, c.dtype, seg, nseg, n_call, sk, sv, w, e, V, nullptr, at<float>(ws, B.dw), int(R),
                                c.d_value, c.accumulate_dv != 0, at<void>(ws, B.aux), &sgd, true),
              "value step");
    }
    return PKM_OK;
  }
  const BwdLayout B = bwd_layout(handle, call_T);
  void* e = at<void>(ws, L.e);
  for (int64_t t0 = 0; t0 < T; t0 += call_T) {
    const int32_t* ci = idx + t0 * R;
    const float* cw = w + t0 * R;
    if (fused)
      PKM_HIP(launch_merge_gather(s, c.dtype, sub_idx, sub_score, T, c.heads, c.topk, c.n_keys2,
                                  1.0f / c.temperature, idx, w, V, y, c.d_value, false, target, e),
              "candidate merge, value gather-sum and reconstruction residual");
    else
      PKM_HIP(launch_gather(s, c.dtype, ci, cw, V, static_cast<char*>(y) + t0 * row_bytes, call_T, int(R), c.d_value,
                            false, static_cast<const char*>(target) + t0 * row_bytes, e),
              "value gather-sum and reconstruction residual");
    VgAdam sgd{};
    sgd.V = V;
    sgd.step_size = lr;
    sgd.sgd = 1;
    PKM_TRY(run_value_grad(handle, s, call_T, ci, cw, e, V, nullptr, at<int32_t>(ws, L.touched),
                           at<int64_t>(ws, L.n_touched), at<float>(ws, B.dw), ws, &sgd, bits, int(streams)));
  }
  return PKM_OK;
}

}  // namespace

pkm_status pkm_fwpkm_chunk(pkm_handle_t handle, void* stream, int64_t T, int64_t streams, const void* q,
                           const void* C, const void* Cp, void* V, const void* target, float lr, void* y, int32_t* idx,
                           float* w, void* ws, size_t ws_bytes) {
  return fwpkm_calls(handle, stream, T, T > 0 ? T : (streams > 0 ? streams : 1), streams, q, C, Cp, V, target, lr, y,
                     idx, w, ws, ws_bytes);
}

pkm_status pkm_fwpkm_chunks(pkm_handle_t handle, void* stream, int64_t T, int64_t call_T, int64_t streams,
                            const void* q, const void* C, const void* Cp, void* V, const void* target, float lr,
                            void* y, int32_t* idx, float* w, void* ws, size_t ws_bytes) {
  return fwpkm_calls(handle, stream, T, call_T, streams, q, C, Cp, V, target, lr, y, idx, w, ws, ws_bytes);
}
