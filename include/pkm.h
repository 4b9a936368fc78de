/*
 * pkm.h - C ABI of the product-key memory (PKM) lookup for AMD Instinct MI355X (gfx950).
 *
 * What is computed (per token t, per head h; all heads share one value table):
 *   q_pre = x W_q^T                       query projection, no bias
 *   q     = BN(q_pre)                     batch-statistics BatchNorm (optional)
 *   q1,q2 = first / second half of head h's dq-wide slice of q
 *   s1[i] = q1 . C[h,i],  s2[j] = q2 . C'[h,j]
 *   I1 = top-k of s1, I2 = top-k of s2    (score descending, lowest index first on ties)
 *   candidates (a,b) in I1 x I2: score s1[I1[a]] + s2[I2[b]], row I1[a]*|C'| + I2[b]
 *   keep the k best candidates (score descending, lowest row first), w = softmax(score / tau)
 *   y[t]  = sum_h sum_s w[t,h,s] * V[row[t,h,s], :]
 * The residual add (x + y) belongs to the caller.
 *
 * Steps, as named by the stage entry points and the kernels' comments:
 *   a1 projection, a2 BatchNorm, a3 sub-key scores, a4 per-half top-k,
 *   a5 candidate merge, top-k and softmax, a6 weighted sum of value rows;
 *   backward: a7 dw and the softmax backward, a8 value-row gradient (touched
 *   rows only), a9 query and sub-key gradients, a10 BatchNorm backward and the
 *   projection gradients (dW_q, dx).
 *
 * Sources (web pages on product-key memory layers):
 *  - "Meta AI 可扩展内存层" (zskr.cn article on Meta AI's scalable memory layers):
 *    section 3.2 (query projection, top-k similarity, softmax, weighted sum),
 *    section 4.3 (two-half lookup and k1 x k2 candidates), section 4.5 (row offset
 *    of pair (i, j)), section 5.3 (value matrix [K1*K2, d], only candidate rows
 *    read), sections 6.1 and 9.2 (only the selected keys and values get gradient),
 *    section 10.1 (bias-free projection, query halves, row i * num_keys_b + j).
 *  - gptget.net summary of arXiv 1907.05242 (product-key memory layer):
 *    method details (C and C' of |C| vectors of dim dq/2; q split into q1, q2;
 *    top-k per half; k best of the candidate set; weighted sum; multi-head;
 *    back-propagation into every parameter), key results (BatchNorm on the
 *    query, h = 4, k = 32), abstract (exact search over the product key set).
 *
 * Conventions (every entry point):
 *  - Pointers named "device" point to device memory the caller owns (for example
 *    torch tensors); the library never allocates device memory and keeps only
 *    immutable host state in the handle.  Row-major, contiguous, 16-byte aligned.
 *  - stream: a hipStream_t passed as void* (NULL = the default stream).  Work is
 *    enqueued asynchronously and the call returns without synchronising; values
 *    written on the device (outputs, *n_touched) are valid once the stream has
 *    reached them.  Kernels run on the device current at the call, which must
 *    be the stream's device and hold (or reach) every device pointer passed.
 *  - Storage dtype (pkm_config.dtype) applies to x, W_q, C, C', V, y, dY, dx and
 *    the saved q.  Arithmetic is fp32 (bf16 storage: bf16 MFMA operands, fp32
 *    accumulation; q is rounded to bf16 after BatchNorm).  All gradients
 *    except dx are fp32.
 *  - Errors: every argument is checked before any HIP call; on failure the call
 *    returns a non-zero pkm_status, touches nothing, and pkm_last_error() gives a
 *    message.  PKM_ERR_HIP reports a failed launch; a device-side fault shows up
 *    at the caller's next synchronisation.  No C++ exception crosses the ABI.
 *  - Threads: a handle's configuration is immutable after pkm_create;
 *    concurrent calls on one handle are safe when they use distinct workspaces
 *    and outputs (pkm_backward serialises only the enqueueing of its side-stream
 *    part).
 *  - Inputs must be finite (not checked on the device).
 */
#ifndef PKM_H_
#define PKM_H_

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef struct pkm_handle_s* pkm_handle_t;

typedef enum {
  PKM_OK = 0,
  PKM_ERR_INVALID_ARG = 1, /* null/misaligned pointer, bad size or config value */
  PKM_ERR_UNSUPPORTED = 2, /* valid but outside what the kernels implement (see limits) */
  PKM_ERR_WORKSPACE = 3,   /* workspace missing or smaller than pkm_workspace_size() */
  PKM_ERR_HIP = 4          /* a HIP runtime call or kernel launch failed */
} pkm_status;

typedef enum { PKM_F32 = 0, PKM_BF16 = 1 } pkm_dtype;
typedef enum { PKM_BN_NONE = 0, PKM_BN_BATCH = 1 } pkm_bn_mode;
/* How the value table V is stored.  PKM_VALUES_FP8 ("Meta AI 可扩展内存层",
 * section 16.3: the value matrix compressed to a low-bit format): row r takes
 * PKM_FP8_ROW_BYTES(d_value) bytes, d_value + 16 rounded up to a multiple of
 * 128 (a row then spans whole 128-byte lines): a 16-byte header whose first 4
 * bytes are the fp32 scale s_r (the other 12 bytes zero), then d_value E4M3
 * codes (1 sign bit, 4 exponent bits with bias 7, 3 mantissa bits, no
 * infinities), then zero bytes up to the row's end; the value is s_r * code.
 * pkm_quantize_values writes such a table.  It is a forward (inference)
 * format: pkm_forward and pkm_stage_gather read it; the entry points that need
 * V in the backward return PKM_ERR_UNSUPPORTED (train a table in the storage
 * dtype and quantize it). */
typedef enum { PKM_VALUES_STORAGE = 0, PKM_VALUES_FP8 = 1 } pkm_value_format;
#define PKM_FP8_ROW_BYTES(d_value) ((((int64_t)(d_value) + 16 + 127) / 128) * 128)
/* Sub-key score.  PKM_SCORE_DOT: s1[i] = q1 . C[h,i] (as above).  PKM_SCORE_IDW
 * ("Fast-weight Product Key Memory", section 2.2: inverse-distance scores):
 * s1[i] = -log ||q1 - C[h,i]||, computed as -1/2 log(max(||q1||^2 - (2 q1 . C[h,i]
 * - ||C[h,i]||^2), 1e-12)) in fp32, likewise s2 against C'; the per-half top-k
 * ranks on 2 q1 . C[h,i] - ||C[h,i]||^2, which orders the sub-keys as the
 * distance does.  The full-key score stays s1 + s2, so the product-key search is
 * still exact.  With IDW, pkm_forward, pkm_stage_score_topk and pkm_fwpkm_chunk
 * score this way; pkm_backward, pkm_backward_adam and pkm_stage_subkey_grad
 * return PKM_ERR_UNSUPPORTED (their score gradients are the dot product's). */
typedef enum { PKM_SCORE_DOT = 0, PKM_SCORE_IDW = 1 } pkm_score_fn;
/* pkm_workspace_size's with_backward: the forward, the backward, or pkm_fwpkm_chunk. */
typedef enum { PKM_WS_FORWARD = 0, PKM_WS_BACKWARD = 1, PKM_WS_FWPKM_CHUNK = 2 } pkm_ws_kind;

/* Layer shape.  pkm_create checks (v = 8 elements for bf16, 4 for fp32 storage,
 * i.e. 16 bytes):
 *   d_in >= 1, d_in % v == 0;  heads >= 1;  d_query >= 2, even, (d_query/2) % v == 0;
 *   1 <= topk <= 32, topk <= n_keys, topk <= n_keys2;  1 <= n_keys, n_keys2 <= 2048;
 *   n_keys * n_keys2 < 2^31;  d_value >= 1, d_value % v == 0, d_value * elem <= 4096 bytes;
 *   temperature > 0;  bn_eps >= 0 (BN_BATCH);
 *   value_format PKM_VALUES_FP8: d_value % 16 == 0 and d_value <= 4096.
 * Per call: T >= 0 (T = 0 is a no-op; the backward then zeroes its gradients)
 * and T * heads * topk <= 2^26 lookups. */
typedef struct {
  int32_t d_in;          /* d: width of x */
  int32_t heads;         /* h */
  int32_t d_query;       /* dq: per-head query width (two halves of dq/2) */
  int32_t n_keys;        /* |C|: sub-keys of the first half, per head */
  int32_t n_keys2;       /* |C'|: sub-keys of the second half, per head */
  int32_t topk;          /* k: per-half top-k and number of selected slots per head */
  int32_t d_value;       /* width of a value row and of y */
  int32_t dtype;         /* pkm_dtype */
  int32_t bn;            /* pkm_bn_mode */
  float bn_eps;          /* BatchNorm epsilon (1e-5) */
  float temperature;     /* tau: w = softmax(score / tau) (1.0) */
  int32_t accumulate_dv; /* pkm_backward: 1 -> dV[r] += g_r, 0 -> dV[r] = g_r (touched rows only) */
  int32_t value_format;  /* pkm_value_format: PKM_VALUES_STORAGE (V in the storage dtype) or PKM_VALUES_FP8 */
  int32_t score_fn;      /* pkm_score_fn: PKM_SCORE_DOT or PKM_SCORE_IDW */
} pkm_config;

/* State the forward saves for the backward; every buffer is caller-allocated device memory. */
typedef struct {
  int32_t* idx;   /* [T, h, k] selected rows, per (t, h) ordered by (score desc, row asc) */
  float* w;       /* [T, h, k] softmax weights, same order */
  void* q;        /* [T, h*dq] storage dtype: the query after BatchNorm (and bf16 rounding) */
  float* q_pre;   /* [T, h*dq] fp32: x W_q^T */
  float* bn_mean; /* [h*dq] batch mean (BN_BATCH; unused and may be NULL with BN_NONE) */
  float* bn_rstd; /* [h*dq] 1/sqrt(var + eps) (BN_BATCH; may be NULL with BN_NONE) */
} pkm_saved;

/* Adam hyper-parameters of the value table's optimizer step (pkm_backward_adam,
 * pkm_stage_value_adam).  "Meta AI 可扩展内存层", section 6.3: moments only for
 * the parameters that received gradient, and a learning rate of the value
 * table's own.  Checked on the host: lr finite >= 0, beta1 and beta2 in [0, 1),
 * eps finite > 0, step >= 1. */
typedef struct {
  float lr;
  float beta1;
  float beta2;
  float eps;
  int64_t step; /* 1-based global count of optimizer steps, this one included (bias correction) */
} pkm_adam;

/* Adam moments kept only for the rows that have received gradient
 * ("Meta AI 可扩展内存层", section 6.3: optimizer state allocated only for the
 * parameters that got gradient), for pkm_backward_adam_rows and
 * pkm_stage_value_adam_rows.  All pointers are caller-allocated device memory.
 *   slot [|C|*|C'|] int32: -1 for a row without moments, else the row of m and
 *     v holding its moments.  Set to -1 everywhere before the first step; the
 *     library writes it (between calls every entry is -1 or a slot below
 *     capacity; a call writes other values transiently).
 *   m, v [capacity, d_value] fp32: the pool; need not be initialised (a row's
 *     first step starts from zero moments and does not read its slot); may be
 *     NULL when capacity is 0.
 *   n_used [1] int64 (8-byte aligned): slots handed out so far; 0 before the
 *     first step.  A call gives the touched rows without a slot, in ascending
 *     row order, the slots n_used, n_used + 1, ...; a row whose slot would be
 *     capacity or more keeps -1 and is not stepped (its V row and the pool are
 *     unchanged), yet n_used counts it: n_used > capacity after a call means
 *     that many rows asked in vain, and the caller should grow the pool.
 *   capacity: rows of m and v, 0 <= capacity <= |C|*|C'| (checked).
 * Entries of slot outside [-1, capacity) are never used as pool rows (such a
 * row is not stepped). */
typedef struct {
  int32_t* slot;
  float* m;
  float* v;
  int64_t* n_used;
  int64_t capacity;
} pkm_adam_rows;

/* Validate cfg and build a handle.  Besides host state, the handle owns one
 * HIP stream (default priority, non-blocking) and two events created on the
 * device current at this call; pkm_backward uses them to run the sub-key
 * gradients beside the projection gradients.  If they cannot be created (no
 * device), pkm_backward runs on the caller's stream alone.  No device memory
 * is allocated.  pkm_destroy releases them. */
pkm_status pkm_create(const pkm_config* cfg, pkm_handle_t* out);
pkm_status pkm_destroy(pkm_handle_t handle);
/* The config the handle was created with. */
pkm_status pkm_get_config(pkm_handle_t handle, pkm_config* out);

/* Device workspace (bytes) that pkm_forward (with_backward = PKM_WS_FORWARD),
 * pkm_backward (PKM_WS_BACKWARD) or pkm_fwpkm_chunk (PKM_WS_FWPKM_CHUNK) needs
 * for T tokens; any other value is PKM_ERR_INVALID_ARG.  The caller allocates it. */
pkm_status pkm_workspace_size(pkm_handle_t handle, int64_t T, int with_backward, size_t* bytes);

/* Forward m(x) for T >= 1 tokens.  Device pointers:
 *   x [T, d_in], Wq [h*dq, d_in] (out x in), C [h, |C|, dq/2], Cp [h, |C'|, dq/2],
 *   V [|C|*|C'|, d_value]: storage dtype.  bn_gamma, bn_beta [h*dq] fp32 (BN_BATCH only).
 *   y [T, d_value] storage dtype (output).  saved: all its buffers are written.
 *   ws: workspace of ws_bytes >= pkm_workspace_size(handle, T, 0). */
pkm_status pkm_forward(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                       const float* bn_gamma, const float* bn_beta, const void* C, const void* Cp,
                       const void* V, void* y, const pkm_saved* saved, void* ws, size_t ws_bytes);

/* pkm_forward for callers that cannot allocate device memory (code under HIP
 * graph capture, tight serving loops, harnesses that forbid hipMalloc): the
 * same kernels and results as pkm_forward, with no ws argument.  The
 * workspace is a static device array of 128 MiB in the library, one copy
 * per device (at most 64 devices), held until the process ends; its device
 * address is looked up on the first call on each device (with that device
 * current).  Nothing is allocated and nothing needs clearing.  T whose
 * pkm_workspace_size(handle, T, 0) exceeds 128 MiB returns PKM_ERR_WORKSPACE
 * (58,872 tokens at h = 4, dq = 512, 1024 sub-keys per half, k = 32).  All calls on one device share the
 * array: calls that overlap in time on one device (different streams, or
 * host threads without ordering between them) race; calls in order on one
 * stream do not.  Other arguments as in pkm_forward. */
pkm_status pkm_forward_noalloc(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                               const float* bn_gamma, const float* bn_beta, const void* C, const void* Cp,
                               const void* V, void* y, const pkm_saved* saved);

/* Backward of sum(dY * y) given the forward's saved state (same T, same inputs).
 * Outputs (device):
 *   dV [|C|*|C'|, d_value] fp32: only touched rows are read/written (accumulate_dv);
 *   touched [T*h*k] int32: the distinct selected rows, ascending, first *n_touched valid;
 *   n_touched: one int64 on the device;
 *   dC [h, |C|, dq/2], dCp [h, |C'|, dq/2], dWq [h*dq, d_in] fp32 (overwritten);
 *   dgamma, dbeta [h*dq] fp32 (BN_BATCH; may be NULL with BN_NONE);
 *   dx [T, d_in] storage dtype, may be NULL (not computed).
 *   ws: workspace of ws_bytes >= pkm_workspace_size(handle, T, 1).
 * On the device current at pkm_create, part of the work (dC, dC') runs on the
 * handle's side stream, forked from and joined back into `stream` with events,
 * so all outputs are complete once `stream` has reached the end of this call
 * (also under stream capture: the side stream joins the capture). */
pkm_status pkm_backward(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                        const void* Wq, const float* bn_gamma, const void* C, const void* Cp,
                        const void* V, const pkm_saved* saved, float* dV, int32_t* touched,
                        int64_t* n_touched, float* dC, float* dCp, float* dWq, float* dgamma,
                        float* dbeta, void* dx, void* ws, size_t ws_bytes);

/* pkm_backward with the value table's optimizer step fused into the value
 * gradient: no dV.  For every touched row r (the rows of saved->idx; all other
 * rows of V, adam_m and adam_v are neither read nor written), with g_r the
 * row's gradient of this call (what pkm_backward would write into dV with
 * accumulate_dv = 0) and t = adam->step:
 *   m_r = beta1 m_r + (1 - beta1) g_r,   v_r = beta2 v_r + (1 - beta2) g_r^2,
 *   V_r = V_r - lr * (m_r / (1 - beta1^t)) / (sqrt(v_r / (1 - beta2^t)) + eps),
 * elementwise in fp32, V_r rounded to the storage dtype.  dw and everything
 * after it use the rows of V before this step.  V [|C|*|C'|, d_value] storage
 * dtype (updated in place); adam_m, adam_v [|C|*|C'|, d_value] fp32 (caller
 * allocated, zero before the first step).  The other arguments, outputs and the
 * workspace are those of pkm_backward; cfg.accumulate_dv is ignored. */
pkm_status pkm_backward_adam(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                             const void* Wq, const float* bn_gamma, const void* C, const void* Cp, void* V,
                             const pkm_saved* saved, float* adam_m, float* adam_v, const pkm_adam* adam,
                             int32_t* touched, int64_t* n_touched, float* dC, float* dCp, float* dWq,
                             float* dgamma, float* dbeta, void* dx, void* ws, size_t ws_bytes);

/* pkm_backward_adam with the moments in the pool of `state` (pkm_adam_rows)
 * instead of dense tables: the same step for every touched row that has or
 * gets a slot; a touched row refused a slot (pool full) is not stepped.  Other
 * arguments, outputs and the workspace as in pkm_backward_adam.  Calls that
 * share a state must be ordered (one stream, or synchronised). */
pkm_status pkm_backward_adam_rows(pkm_handle_t handle, void* stream, int64_t T, const void* dY, const void* x,
                                  const void* Wq, const float* bn_gamma, const void* C, const void* Cp, void* V,
                                  const pkm_saved* saved, const pkm_adam_rows* state, const pkm_adam* adam,
                                  int32_t* touched, int64_t* n_touched, float* dC, float* dCp, float* dWq,
                                  float* dgamma, float* dbeta, void* dx, void* ws, size_t ws_bytes);

const char* pkm_status_string(pkm_status s);
/* Message of the last failed call on this thread ("" if none). */
const char* pkm_last_error(void);

/* ---------------------------------------------------------------------------
 * Stage entry points: each launches exactly the kernels the full calls launch
 * for one step, so every step can be checked on its own inputs.
 * ------------------------------------------------------------------------- */

/* Steps a1-a2: q_pre = x W_q^T, batch statistics, q = BN(q_pre) rounded to storage.
 * Writes saved->q_pre, saved->q, saved->bn_mean, saved->bn_rstd (BN_BATCH).
 * ws >= pkm_workspace_size(handle, T, 0). */
pkm_status pkm_stage_query(pkm_handle_t handle, void* stream, int64_t T, const void* x, const void* Wq,
                           const float* bn_gamma, const float* bn_beta, const pkm_saved* saved,
                           void* ws, size_t ws_bytes);

/* Steps a3-a4: per head and half, scores of q's half against C (C') and the top-k.
 * q [T, h*dq] storage dtype.  Outputs sub_idx int32 and sub_score fp32, both
 * [T, h, 2, k]: [..., 0, :] from C, [..., 1, :] from C', each ordered by
 * (score desc, index asc).  ws >= pkm_workspace_size(handle, T, 0) (holds the
 * sub-keys repacked for the matrix cores). */
pkm_status pkm_stage_score_topk(pkm_handle_t handle, void* stream, int64_t T, const void* q,
                                const void* C, const void* Cp, int32_t* sub_idx, float* sub_score,
                                void* ws, size_t ws_bytes);

/* Step a5: from sorted per-half lists [T, h, 2, k] (as written by the stage
 * above), the k best of the k x k candidates and their softmax weights:
 * idx int32 and w fp32 [T, h, k]; score (may be NULL) fp32 [T, h, k] gets the
 * selected full-key scores. */
pkm_status pkm_stage_merge_softmax(pkm_handle_t handle, void* stream, int64_t T,
                                   const int32_t* sub_idx, const float* sub_score, int32_t* idx,
                                   float* w, float* score);

/* Step a6: y[t] = sum over (h, s) of w[t,h,s] V[idx[t,h,s]].  idx and w [T, h, k];
 * every idx must lie in [0, |C|*|C'|) (not checked on the device). */
pkm_status pkm_stage_gather(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                            const float* w, const void* V, void* y);

/* Steps a7 (dw) and a8: rows of idx sorted (stable), then per touched row r:
 * dw[c] = <dY[t(c)], V[r]> for every lookup c with idx[c] == r, and
 * dV[r] (+)= sum_c w[c] dY[t(c)].  dw [T, h, k] fp32; dV, touched, n_touched as
 * in pkm_backward; every idx must lie in [0, |C|*|C'|) (not checked on the
 * device).  ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_value_grad(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                const float* w, const void* dY, const void* V, float* dV,
                                int32_t* touched, int64_t* n_touched, float* dw, void* ws,
                                size_t ws_bytes);

/* Steps a7 (dw) and a8 with the Adam step of pkm_backward_adam in place of
 * dV: dw [T, h, k] fp32 from the rows of V before the step; V, adam_m, adam_v
 * updated at the touched rows; touched, n_touched as in pkm_backward; every
 * idx must lie in [0, |C|*|C'|) (not checked on the device).
 * ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_value_adam(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                const float* w, const void* dY, void* V, float* adam_m, float* adam_v,
                                const pkm_adam* adam, int32_t* touched, int64_t* n_touched, float* dw,
                                void* ws, size_t ws_bytes);

/* Monitoring signals of a batch's selection ("Meta AI 可扩展内存层", section 11.2:
 * codebook hit distribution, per-sub-key hit counts, candidate softmax entropy;
 * section 9.3: per-sub-key hits and gradient density; product-key paper summary,
 * key results: memory usage, the share of slots in use).  From idx, w [T, h, k]
 * (as the forward saves them), all outputs on the device:
 *   hits_c [h, |C|], hits_cp [h, |C'|] int32: selected slots of head h whose row
 *     has first-half sub-key i (row / |C'| == i), second-half sub-key j (row % |C'|);
 *   used [1 + h] int64 (8-byte aligned): distinct rows over all heads, then per head;
 *   entropy [T, h] fp32 (may be NULL): -sum_s w log w (w = 0 terms count 0);
 *   entropy_sum [1] fp64 (may be NULL, 8-byte aligned): the sum of entropy over
 *     (t, h), in a fixed order.
 * Integer outputs are exact; rows outside [0, |C|*|C'|) are not counted.
 * ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_diagnostics(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx, const float* w,
                           int32_t* hits_c, int32_t* hits_cp, int64_t* used, float* entropy, double* entropy_sum,
                           void* ws, size_t ws_bytes);

/* The fp8 value table of PKM_VALUES_FP8 from rows in the storage dtype: for
 * each of the `rows` rows of V_src [rows, d_value], s_r = max_j |V_src[r, j]| / 448
 * and code j = the E4M3 value nearest to V_src[r, j] * (448 / max_j |V_src[r, j]|)
 * (ties to the even code; scale, factor and product rounded to fp32); a zero
 * row gets s_r = 0 and zero codes.  V_fp8: rows * PKM_FP8_ROW_BYTES(d_value)
 * bytes, layout as described at pkm_value_format (every byte is written).  The handle must have value_format =
 * PKM_VALUES_FP8.  rows >= 0. */
pkm_status pkm_quantize_values(pkm_handle_t handle, void* stream, const void* V_src, int64_t rows, void* V_fp8);

/* Step a8's grouping alone: the lookups of idx [T, h, k] stably sorted by row,
 * written into the workspace (for pkm_stage_value_grad_grouped), plus touched
 * and *n_touched as in pkm_backward; every idx must lie in [0, |C|*|C'|) (not
 * checked on the device).  ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_row_groups(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                int32_t* touched, int64_t* n_touched, void* ws, size_t ws_bytes);

/* Steps a7 (dw) and a8 on a grouping already in ws (pkm_stage_row_groups with
 * the same handle, T, idx and n_touched): launches the value-gradient kernel only.
 * w, dY, V, dV, dw as in pkm_stage_value_grad; n_touched is read on the device. */
pkm_status pkm_stage_value_grad_grouped(pkm_handle_t handle, void* stream, int64_t T, const float* w,
                                        const void* dY, const void* V, float* dV, float* dw,
                                        const int64_t* n_touched, void* ws, size_t ws_bytes);

/* pkm_stage_value_adam on a grouping already in ws (pkm_stage_row_groups with
 * the same handle, T, idx and n_touched): launches the value-gradient kernel
 * with the Adam step only.  Arguments as in pkm_stage_value_adam. */
pkm_status pkm_stage_value_adam_grouped(pkm_handle_t handle, void* stream, int64_t T, const float* w,
                                        const void* dY, void* V, float* adam_m, float* adam_v,
                                        const pkm_adam* adam, float* dw, const int64_t* n_touched, void* ws,
                                        size_t ws_bytes);

/* pkm_stage_value_adam with the moments in the pool of `state` (as in
 * pkm_backward_adam_rows): the grouping, the slot hand-out for the touched
 * rows without one, then the value-gradient kernel with the Adam step.  Every
 * idx must lie in [0, |C|*|C'|) (not checked on the device).
 * ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_value_adam_rows(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                     const float* w, const void* dY, void* V, const pkm_adam_rows* state,
                                     const pkm_adam* adam, int32_t* touched, int64_t* n_touched, float* dw,
                                     void* ws, size_t ws_bytes);

/* Steps a7 (softmax backward) and a9: ds = w (dw - sum_s w dw) / tau; then
 * dq[t, h*dq] fp32 (both halves of each head) and dC, dCp (overwritten) through
 * the selected sub-keys only.  q is the saved query (storage dtype); every idx
 * must lie in [0, |C|*|C'|) (not checked on the device).
 * ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_subkey_grad(pkm_handle_t handle, void* stream, int64_t T, const int32_t* idx,
                                 const float* w, const float* dw, const void* q, const void* C,
                                 const void* Cp, float* dq, float* dC, float* dCp, void* ws,
                                 size_t ws_bytes);

/* Step a10: BatchNorm backward (batch statistics) and the projection's
 * gradients: dgamma, dbeta [h*dq], dWq [h*dq, d_in] fp32, dx [T, d_in] storage
 * dtype (may be NULL).  dq [T, h*dq] fp32; saved->q_pre/bn_mean/bn_rstd as
 * written by the forward.  ws >= pkm_workspace_size(handle, T, 1). */
pkm_status pkm_stage_query_grad(pkm_handle_t handle, void* stream, int64_t T, const float* dq,
                                const void* x, const void* Wq, const float* bn_gamma,
                                const pkm_saved* saved, float* dWq, float* dgamma, float* dbeta,
                                void* dx, void* ws, size_t ws_bytes);

/* One chunk of FwPKM memorization ("Fast-weight Product Key Memory", sections
 * 2.1 and 2.2: the value table is a fast weight that the layer itself writes
 * while it reads, by a gradient step on a local reconstruction loss toward the
 * caller's lookahead targets).  The call holds one chunk of each of `streams`
 * independent streams (a batch of sequences, each with its own value table;
 * the sub-keys are shared): T = streams * chunk tokens, stream b's tokens are
 * rows [b*T/streams, (b+1)*T/streams) of q, target and y, and its table is rows
 * [b*|C|*|C'|, (b+1)*|C|*|C'|) of V.  For every token, with the handle's IDW
 * scores (score_fn must be PKM_SCORE_IDW, else PKM_ERR_UNSUPPORTED;
 * value_format must be PKM_VALUES_STORAGE):
 *   idx, w  = the selection of q (as pkm_stage_score_topk + pkm_stage_merge_softmax),
 *             idx as rows of V (stream b's rows offset by b*|C|*|C'|);
 *   y[t]    = sum over (h, s) of w V[idx] from V BEFORE the write, rounded to storage;
 *   e[t]    = y[t] - target[t], rounded to storage (the gradient of 1/2 ||y - target||^2);
 *   V[r]    = V[r] - lr * sum over the lookups c of r of w[c] e[t(c)], fp32, rounded
 *             to storage, for every selected row r (no other row is read or written).
 * The per-row sums run in a fixed order, so the result is deterministic.
 * Device pointers: q [T, h*dq], C [h, |C|, dq/2], Cp [h, |C'|, dq/2], V
 * [streams*|C|*|C'|, d_value] (updated in place), target and y [T, d_value]:
 * storage dtype; idx int32 and w fp32 [T, h, k] (outputs, ordered as in
 * pkm_saved).  streams >= 1 dividing T, streams*|C|*|C'| < 2^31; lr finite >= 0.
 * ws >= pkm_workspace_size(handle, T, PKM_WS_FWPKM_CHUNK).  Chunks that follow
 * one another are calls that follow one another on the stream. */
pkm_status pkm_fwpkm_chunk(pkm_handle_t handle, void* stream, int64_t T, int64_t streams, const void* q,
                           const void* C, const void* Cp, void* V, const void* target, float lr, void* y,
                           int32_t* idx, float* w, void* ws, size_t ws_bytes);

/* A run of memorization calls in one: the same as calling pkm_fwpkm_chunk on
 * the consecutive slices of call_T tokens of q, target, y, idx and w (slice j
 * is rows [j*call_T, (j+1)*call_T)), in order, with the same streams, V and lr;
 * the results are those calls' results, bit for bit.  For a stream whose
 * queries are all known before it is memorized (a prompt, a document): the
 * selection reads only q, C and C', not V ("Fast-weight Product Key Memory",
 * section 2.2: memorization writes the value table only), so it runs once over
 * all T tokens, as does (when every slice's streams fit one workgroup each)
 * the grouping of the slices' lookups by row; each slice then runs only its
 * gather and its value step.
 * T a multiple of call_T, call_T a multiple of streams; other arguments as in
 * pkm_fwpkm_chunk, with T tokens.  ws >= pkm_workspace_size(handle, T,
 * PKM_WS_FWPKM_CHUNK). */
pkm_status pkm_fwpkm_chunks(pkm_handle_t handle, void* stream, int64_t T, int64_t call_T, int64_t streams,
                            const void* q, const void* C, const void* Cp, void* V, const void* target, float lr,
                            void* y, int32_t* idx, float* w, void* ws, size_t ws_bytes);

#ifdef __cplusplus
}
#endif

#endif /* PKM_H_ */
