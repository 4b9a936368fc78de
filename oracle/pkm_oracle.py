"""Plain fp64 CPU oracle of the product-key memory (PKM) lookup.

TEST INFRASTRUCTURE ONLY.  Nothing on the product path may import, call or
execute this module: only the tests, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py`` use it.  It shares no code with the HIP
library and imports nothing from it; its inputs come from ``pkm_inputs``.

Every step is the plain definition, in float64, written from the pages:

* [Blog] "Meta AI 可扩展内存层" (zskr.cn long-form article on Meta AI's
  scalable memory layers): §3.2 (layer = query projection, top-k similarity,
  softmax, weighted sum of values), §4.3 (two-half product-key lookup: top-k
  per half, k1*k2 Cartesian candidates, full-key score = sum of the two half
  scores), §4.5 (value row of pair (i, j) found by offset), §5.3 (values are a
  [K1*K2, d] matrix read only at the candidate rows), §6.1 and §9.2 (only the
  selected keys and values receive gradient), §10.1 (simplified module: query
  projection without bias, query split into a first and second half, row
  ``i * num_keys_b + j``).
* [PKM-summary] gptget.net summary of arXiv 1907.05242 (product-key memory
  layer): "方法论" and "方法详解" (sub-key sets C and C', each |C| vectors of
  dim dq/2; q(x) split into q1, q2; top-k in each half; the candidate set is
  searched again for the k best keys; weighted sum of the values; multiple
  heads; all parameters trained by back-propagation), "关键结果" (BatchNorm on
  the query, h = 4, k = 32), abstract (the product-key search is exact).

Readings where the pages leave a step open:
heads each own a W_q slice, a C and a C'; they share V and their outputs are
summed.  BatchNorm uses the batch statistics of the call (biased variance,
eps), no bias on the projection, softmax of the raw full-key scores divided
by a temperature tau (default 1), ties broken by lowest index, the residual
add is left to the caller.  For bf16 storage the BatchNorm output q is
rounded to the nearest bf16 (the value the scores are computed from) and the
rounding is passed straight through in the backward.

Beyond the lookup, ``sparse_adam_rows`` is the optimizer step on the touched
value rows that [Blog] §6.3 describes (moments only for rows with gradient;
``adam_rows_state_step`` keeps them in a pool of slots handed out on a row's
first gradient),
``diagnostics`` the monitoring signals of [Blog] §9.3 and §11.2, and
``quantize_rows_fp8`` / ``e4m3_*`` the fp8 value storage of [Blog] §16.3,
``subkey_scores_idw`` and ``fwpkm_chunk`` the fast-weight memorization of the
FwPKM page (fourth source page: "Fast-weight Product Key Memory" summary,
sections 2.1-2.2).

Parity pins (all in ``tests/test_oracle_pins.py``): brute force over every
full key, integer-valued exact ties, numpy cross-checks against dense
formulations, closed forms of BatchNorm and softmax, finite differences of
every gradient, and conservation identities.  No function here is left
unpinned.
"""
from __future__ import annotations

import numpy as np

F32 = "f32"
BF16 = "bf16"
F64 = "f64"   # exact arithmetic (finite-difference checks): nothing is rounded


# ---------------------------------------------------------------------------
# storage formats
# ---------------------------------------------------------------------------
def decode(a: np.ndarray, dtype: str) -> np.ndarray:
    """Stored tensor -> exact float64 values (bf16 is given as uint16 bits)."""
    if dtype == BF16:
        u = np.ascontiguousarray(a).astype(np.uint32) << np.uint32(16)
        return u.view(np.float32).astype(np.float64)
    return np.asarray(a, dtype=np.float64)


def round_to_bf16(v: np.ndarray) -> np.ndarray:
    """Nearest bf16 value (8 significant bits, ties to even), as float64.

    v = m * 2**e with 0.5 <= |m| < 1; a bf16 keeps 8 significant bits, so the
    spacing around v is 2**(e - 8) (never below the fp32/bf16 subnormal
    spacing 2**-133).  ``np.rint`` rounds half to even.
    """
    v = np.asarray(v, dtype=np.float64)
    _, e = np.frexp(v)
    step = np.ldexp(1.0, np.maximum(e - 8, -133))
    return np.rint(v / step) * step


def round_to_storage(v: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == BF16:
        return round_to_bf16(v)
    if dtype == F64:
        return np.asarray(v, dtype=np.float64)
    return np.asarray(v, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# a1, a2: query network q(x) = BN(W_q x)
# ---------------------------------------------------------------------------
def project(x: np.ndarray, Wq: np.ndarray) -> np.ndarray:
    """q_pre = x W_q^T, no bias ([Blog] §3.2 and §10.1; [PKM-summary] method details)."""
    return x @ Wq.T


def batchnorm_forward(q_pre: np.ndarray, gamma: np.ndarray, beta: np.ndarray, eps: float):
    """Per-feature batch normalisation over the tokens of the call ([PKM-summary] key results).

    mean and biased variance over the batch; xhat = (q_pre - mean) / sqrt(var + eps);
    q = gamma * xhat + beta.
    """
    mean = q_pre.mean(axis=0)
    var = ((q_pre - mean) ** 2).mean(axis=0)
    xhat = (q_pre - mean) / np.sqrt(var + eps)
    return gamma * xhat + beta, mean, var, xhat


# ---------------------------------------------------------------------------
# a3, a4: half-query scores against C and C', top-k per half
# ---------------------------------------------------------------------------
def split_heads(q: np.ndarray, heads: int, dq: int):
    """q [T, h*dq] -> (q1, q2), each [T, h, dq/2]: first and second half of every head's query."""
    T = q.shape[0]
    qh = q.reshape(T, heads, dq)
    return qh[:, :, : dq // 2], qh[:, :, dq // 2:]


def subkey_scores(q1: np.ndarray, q2: np.ndarray, C: np.ndarray, Cp: np.ndarray):
    """s1[t,h,i] = q1[t,h].C[h,i]; s2[t,h,j] = q2[t,h].C'[h,j] ([Blog] §4.3; [PKM-summary] method details)."""
    s1 = np.einsum("thd,hid->thi", q1, C, optimize=True)
    s2 = np.einsum("thd,hjd->thj", q2, Cp, optimize=True)
    return s1, s2


IDW_FLOOR = 1e-12  # squared distances below this count as this (a query on a key)


def subkey_scores_idw(q1: np.ndarray, q2: np.ndarray, C: np.ndarray, Cp: np.ndarray):
    """s1[t,h,i] = -log ||q1[t,h] - C[h,i]||, likewise s2 against C' (FwPKM page, section 2.2: the
    negative log of the Euclidean distance replaces the dot product).  Squared distances are floored
    at IDW_FLOOR; computed from the differences, float64."""
    def idw(qh, K):
        d2 = ((qh[:, :, None, :] - K[None, :, :, :]) ** 2).sum(-1)
        return -0.5 * np.log(np.maximum(d2, IDW_FLOOR))
    return idw(q1, C), idw(q2, Cp)


def topk_sorted(s: np.ndarray, k: int):
    """Indices and values of the k largest entries along the last axis.

    Order: score descending, index ascending among equal scores (a stable sort
    of -s; -0.0 and +0.0 compare equal, so they are ordered by index).
    """
    order = np.argsort(-s, axis=-1, kind="stable")[..., :k]
    return order, np.take_along_axis(s, order, axis=-1)


# ---------------------------------------------------------------------------
# a5: k x k candidates, top-k of them, softmax
# ---------------------------------------------------------------------------
def candidates(i1, v1, i2, v2, n_keys2: int):
    """All k1*k2 pairs (a, b): full-key score v1[a] + v2[b], row i1[a]*|C'| + i2[b].

    ([Blog] §4.3 and §4.5; §10.1's combined index.)  Flattened a-major.
    """
    sc = v1[..., :, None] + v2[..., None, :]
    rows = i1[..., :, None].astype(np.int64) * n_keys2 + i2[..., None, :].astype(np.int64)
    shp = sc.shape[:-2] + (sc.shape[-2] * sc.shape[-1],)
    return sc.reshape(shp), rows.reshape(shp)


def select_topk(scores: np.ndarray, rows: np.ndarray, k: int):
    """The k best candidates by (score descending, row ascending) ([PKM-summary] method details)."""
    order = np.lexsort((rows, -scores), axis=-1)[..., :k]
    return np.take_along_axis(rows, order, axis=-1), np.take_along_axis(scores, order, axis=-1)


def softmax(s: np.ndarray, tau: float) -> np.ndarray:
    """w = exp(s/tau) / sum exp(s/tau) over the selected keys ([Blog] §3.2, §5.3)."""
    z = s / tau
    z = z - z.max(axis=-1, keepdims=True)
    e = np.exp(z)
    return e / e.sum(axis=-1, keepdims=True)


# ---------------------------------------------------------------------------
# a6: softmax-weighted sum of value rows, heads summed
# ---------------------------------------------------------------------------
def gather_sum(rows: np.ndarray, w: np.ndarray, V: np.ndarray, v_dtype: str, chunk: int = 256) -> np.ndarray:
    """y[t] = sum_h sum_s w[t,h,s] V[rows[t,h,s]] ([Blog] §5.3), float64.

    ``V`` is the stored value table (decoded row by row, only at the used rows).
    """
    T = rows.shape[0]
    y = np.zeros((T, V.shape[1]), dtype=np.float64)
    for lo in range(0, T, chunk):
        hi = min(T, lo + chunk)
        r = rows[lo:hi].reshape(hi - lo, -1)
        vv = decode(V[r.reshape(-1)], v_dtype).reshape(hi - lo, r.shape[1], -1)
        y[lo:hi] = np.einsum("ts,tsd->td", w[lo:hi].reshape(hi - lo, -1), vv)
    return y


# ---------------------------------------------------------------------------
# the whole forward
# ---------------------------------------------------------------------------
def query(cfg, inp: dict):
    """q_pre, BN state and the query q in storage precision, for all T tokens."""
    x = decode(inp["x"], cfg.dtype)
    Wq = decode(inp["Wq"], cfg.dtype)
    q_pre = project(x, Wq)
    if cfg.bn:
        qn, mean, var, xhat = batchnorm_forward(q_pre, inp["gamma"].astype(np.float64),
                                                inp["beta"].astype(np.float64), cfg.bn_eps)
    else:
        qn, mean, var, xhat = q_pre, None, None, None
    q = round_to_storage(qn, cfg.dtype)
    return {"q_pre": q_pre, "mean": mean, "var": var, "xhat": xhat, "q": q}


def lookup(cfg, q: np.ndarray, C: np.ndarray, Cp: np.ndarray, keep_tables: bool = False, score: str = "dot"):
    """Product-key selection and weights for the tokens whose queries are ``q`` [n, h*dq].

    Returns rows/scores/w [n, h, k] (rows ordered by score desc, row asc), the
    per-half top-k lists and, for the gap rule, the per-half (k+1)-th values.
    ``score``: "dot" (sub-key dot products) or "idw" (negative log distances,
    subkey_scores_idw); either way a full key scores the sum of its halves.
    """
    k = cfg.topk
    q1, q2 = split_heads(q, cfg.heads, cfg.dq)
    s1, s2 = (subkey_scores_idw if score == "idw" else subkey_scores)(q1, q2, C, Cp)
    k1 = min(k + 1, s1.shape[-1])
    k2 = min(k + 1, s2.shape[-1])
    i1, v1 = topk_sorted(s1, k1)
    i2, v2 = topk_sorted(s2, k2)
    sc, rw = candidates(i1[..., :k], v1[..., :k], i2[..., :k], v2[..., :k], cfg.n_keys2)
    rows, scores = select_topk(sc, rw, k)
    w = softmax(scores, cfg.temperature)
    # the k+1 best full keys (same exactness argument with k+1 per half), for near-tie checks
    kk = min(k + 1, k1 * k2)
    sck, rwk = candidates(i1, v1, i2, v2, cfg.n_keys2)
    rows_k1, scores_k1 = select_topk(sck, rwk, kk)
    out = {"rows": rows, "scores": scores, "w": w, "rows_k1": rows_k1, "scores_k1": scores_k1,
           "sub_idx1": i1[..., :k], "sub_val1": v1[..., :k],
           "sub_idx2": i2[..., :k], "sub_val2": v2[..., :k],
           "sub_next1": v1[..., k] if k1 > k else None,
           "sub_next2": v2[..., k] if k2 > k else None}
    if keep_tables:
        out["s1"], out["s2"] = s1, s2
    return out


def forward(cfg, inp: dict, tokens=None, keep_tables: bool = False, chunk: int = 1024, score: str = "dot"):
    """The memory output m(x) (no residual) for ``tokens`` (default all).

    BatchNorm statistics always use all T tokens of the call.  ``score`` as in lookup.
    """
    qs = query(cfg, inp)
    C = decode(inp["C"], cfg.dtype)
    Cp = decode(inp["Cp"], cfg.dtype)
    tok = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    parts = []
    for lo in range(0, len(tok), chunk):
        parts.append(lookup(cfg, qs["q"][tok[lo:lo + chunk]], C, Cp, keep_tables, score))
    sel = {key: (None if parts[0][key] is None else np.concatenate([p[key] for p in parts]))
           for key in parts[0]}
    y = gather_sum(sel["rows"], sel["w"], inp["V"], cfg.dtype)
    out = dict(qs)
    out.update(sel)
    out["tokens"] = tok
    out["y"] = y
    out["y_stored"] = round_to_storage(y, cfg.dtype)
    return out


def brute_force_select(cfg, q: np.ndarray, C: np.ndarray, Cp: np.ndarray):
    """Exact top-k over every full key [C[h,i]; C'[h,j]] (row i*|C'|+j), tiny inputs only.

    The abstract of [PKM-summary] states that product-key search returns the
    exact nearest neighbours; this is the search it must agree with.
    """
    h, nk, half = C.shape
    nk2 = Cp.shape[1]
    keys = np.concatenate([np.repeat(C, nk2, axis=1), np.tile(Cp, (1, nk, 1))], axis=2)  # [h, nk*nk2, dq]
    qh = q.reshape(q.shape[0], h, 2 * half)
    full = np.einsum("thd,hrd->thr", qh, keys)
    rows = np.broadcast_to(np.arange(nk * nk2), full.shape)
    return select_topk(full, rows, cfg.topk)


# ---------------------------------------------------------------------------
# backward (a7 - a10)
# ---------------------------------------------------------------------------
def value_grad_rows(rows: np.ndarray, w: np.ndarray, dY: np.ndarray, y_dtype: str, which: np.ndarray):
    """dV[r] = sum over lookups (t,h,s) with rows[t,h,s] == r of w[t,h,s] dY[t], for r in ``which``.

    ([Blog] §6.1: only activated value rows accumulate gradient.)  Returns a
    [len(which), d] float64 array.
    """
    flat = rows.reshape(-1)
    T = rows.shape[0]
    per_tok = flat.size // T
    order = np.argsort(flat, kind="stable")
    srt = flat[order]
    out = np.zeros((len(which), dY.shape[1]), dtype=np.float64)
    for n, r in enumerate(np.asarray(which)):
        lo, hi = np.searchsorted(srt, r, "left"), np.searchsorted(srt, r, "right")
        c = order[lo:hi]
        if c.size:
            out[n] = (w.reshape(-1)[c][:, None] * decode(dY[c // per_tok], y_dtype)).sum(axis=0)
    return out


def value_grad_dense(rows: np.ndarray, w: np.ndarray, dY: np.ndarray, y_dtype: str, n_rows: int) -> np.ndarray:
    """Dense dV [n_rows, d] by scatter-add of w * dY[t] (small shapes only)."""
    T = rows.shape[0]
    per_tok = rows.size // T
    dV = np.zeros((n_rows, dY.shape[1]), dtype=np.float64)
    dYf = decode(dY, y_dtype)
    flat = rows.reshape(-1)
    wf = w.reshape(-1)
    step = 1 << 16
    for lo in range(0, flat.size, step):
        c = np.arange(lo, min(flat.size, lo + step))
        np.add.at(dV, flat[c], wf[c][:, None] * dYf[c // per_tok])
    return dV


def sparse_adam_rows(V_rows: np.ndarray, m_rows: np.ndarray, v_rows: np.ndarray, g: np.ndarray, lr: float,
                     beta1: float, beta2: float, eps: float, step: int, v_dtype: str):
    """One Adam step on the value rows that received gradient in this step.

    ([Blog] §6.3: the optimizer keeps first and second moments only for the
    parameters that actually got gradient, and the value table gets its own
    learning rate; §6.1: only the activated value rows have gradient.)
    Inputs are the touched rows only: their current values ``V_rows`` (stored
    tensor, decoded here), moments ``m_rows``, ``v_rows`` and this step's
    gradient ``g`` (all [n, d]).  Rows that got no gradient are not passed and
    keep value and moments.  Readings: Adam's bias corrections use the global
    step count ``step`` (1 for the first step), and the stored value is rounded
    to the storage type after the update.  Returns (V', m', v') in float64,
    V' holding storage-precision values.
    """
    g = np.asarray(g, dtype=np.float64)
    m1 = beta1 * np.asarray(m_rows, dtype=np.float64) + (1.0 - beta1) * g
    v1 = beta2 * np.asarray(v_rows, dtype=np.float64) + (1.0 - beta2) * g * g
    m_hat = m1 / (1.0 - beta1 ** step)
    v_hat = v1 / (1.0 - beta2 ** step)
    V1 = decode(V_rows, v_dtype) - lr * m_hat / (np.sqrt(v_hat) + eps)
    return round_to_storage(V1, v_dtype), m1, v1


def adam_rows_state_step(touched: np.ndarray, slot: np.ndarray, M: np.ndarray, Vm: np.ndarray, n_used: int,
                         capacity: int, V_rows: np.ndarray, g: np.ndarray, lr: float, beta1: float, beta2: float,
                         eps: float, step: int, v_dtype: str):
    """``sparse_adam_rows`` with the moments held only for rows that have received gradient.

    ([Blog] §6.3: optimizer state is allocated only for the parameters that got
    gradient.)  Readings: the state is a slot map ``slot`` [n_rows] (-1: the row
    has no moments yet) and a pool of ``capacity`` moment rows ``M``, ``Vm``
    [capacity, d]; ``n_used`` slots are handed out.  The rows of ``touched``
    (ascending, this step's rows with gradient) that have no slot take the
    next slots in ascending row order: the i-th of them (from 0) gets slot
    n_used + i.  One whose slot would be capacity or more keeps -1 and is not
    stepped (its value and state unchanged); ``n_used`` still counts it, so a
    result above ``capacity`` reports the shortfall.  A row's first step starts
    from zero moments, so every stepped row follows ``sparse_adam_rows``.
    ``V_rows``, ``g``: [U, d] the touched rows' stored values and gradients.
    Returns (value rows [U, d] after the step, float64 storage values; slot map;
    M; Vm; n_used; stepped [U] bool).
    """
    touched = np.asarray(touched, dtype=np.int64)
    slot = np.array(slot, dtype=np.int64)
    M = np.array(M, dtype=np.float64)
    Vm = np.array(Vm, dtype=np.float64)
    new = slot[touched] == -1
    s_new = n_used + np.cumsum(new) - 1              # slot of each new row, in row order
    granted = new & (s_new < capacity)
    slot[touched[granted]] = s_new[granted]
    stepped = ~new | granted
    out = decode(V_rows, v_dtype).copy()
    s = slot[touched[stepped]]
    fresh = new[stepped][:, None]
    m0 = np.where(fresh, 0.0, M[s])
    v0 = np.where(fresh, 0.0, Vm[s])
    V1, m1, v1 = sparse_adam_rows(np.asarray(V_rows)[stepped], m0, v0, np.asarray(g)[stepped], lr, beta1, beta2,
                                  eps, step, v_dtype)
    out[stepped] = V1
    M[s] = m1
    Vm[s] = v1
    return out, slot, M, Vm, int(n_used + new.sum()), stepped


# ---------------------------------------------------------------------------
# fp8 value storage ([Blog] §16.3: the value table compressed to a low-bit
# format with little loss of retrieval quality)
# ---------------------------------------------------------------------------
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Values of fp8 E4M3 codes (1 sign, 4 exponent bits with bias 7, 3 mantissa
    bits; exponent 0 is subnormal, exponent 15 with mantissa 7 is NaN, no
    infinities), float64."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * 2.0 ** (e - 7))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest E4M3 code of each finite value (ties to the even code), saturated
    at +-448.  Brute force over the 254 finite codes: the candidates are sorted by
    value and the nearest found with a search; an exact tie takes the code with
    a zero last mantissa bit."""
    finite = np.array([c for c in range(256) if not np.isnan(e4m3_decode(np.array([c]))[0])], dtype=np.int64)
    vals = e4m3_decode(finite)
    pos = finite[(vals >= 0) & ~((vals == 0) & (finite == 0x80))]       # +0 .. 448
    pv = e4m3_decode(pos)
    order = np.argsort(pv)
    pos, pv = pos[order], pv[order]
    a = np.minimum(np.abs(np.asarray(x, dtype=np.float64)), E4M3_MAX)
    i = np.clip(np.searchsorted(pv, a), 1, len(pv) - 1)
    lo, hi = pv[i - 1], pv[i]
    d_lo, d_hi = a - lo, hi - a
    take_hi = (d_hi < d_lo) | ((d_hi == d_lo) & ((pos[i] & 1) == 0))
    code = np.where(take_hi, pos[i], pos[i - 1])
    code = np.where(a == 0, 0, code)
    neg = np.signbit(np.asarray(x, dtype=np.float64)) & (code != 0)
    return (code | np.where(neg, 0x80, 0)).astype(np.uint8)


def quantize_rows_fp8(V: np.ndarray, v_dtype: str):
    """Per-row fp8 storage of a value table: scale s_r = max_j |V[r, j]| / 448 and
    codes c = E4M3(V[r, j] * (448 / max_j |V[r, j]|)); a zero row gets s = 0 and
    zero codes.  The scale, its reciprocal factor and the product are rounded to
    fp32, as the library computes them (they decide the integer codes).  Returns
    (scales fp32 [n], codes uint8 [n, d])."""
    Vf = decode(V, v_dtype).astype(np.float32)
    mx = np.abs(Vf).max(axis=1)
    with np.errstate(divide="ignore", invalid="ignore"):
        scale = np.where(mx > 0, mx / np.float32(E4M3_MAX), np.float32(0)).astype(np.float32)
        inv = np.where(mx > 0, np.float32(E4M3_MAX) / mx, np.float32(0)).astype(np.float32)
    q = (Vf * inv[:, None]).astype(np.float32)
    return scale, e4m3_encode(q)


def dequantize_rows_fp8(scale: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """V[r, j] = s_r * value(c[r, j]), float64."""
    return np.asarray(scale, dtype=np.float64)[:, None] * e4m3_decode(codes)


def fwpkm_chunk(cfg, q: np.ndarray, C: np.ndarray, Cp: np.ndarray, V: np.ndarray, target: np.ndarray, lr: float,
                dense: bool = True):
    """One chunk of FwPKM memorization (FwPKM page, sections 2.1-2.2: the value table is a fast weight,
    written during inference by gradient descent on a local reconstruction loss toward lookahead
    targets v_{t+1}; sparse retrieval with IDW scores).

    Readings: the call's queries ``q`` [T, h*dq] (storage values) and targets [T, d_v] (the caller's
    v_{t+1}) are given; lookup with IDW scores; y = the weighted sum of the rows read before the write,
    stored in the storage dtype; loss 1/2 sum_t ||y_t - target_t||^2 with the residual e = y - target
    also in the storage dtype (as an upstream gradient is); only the value rows are written:
    V[r] <- V[r] - lr * sum over the lookups of r of w * e_t, rounded to storage.  Returns
    (y as stored, V after the write, the lookup dict), float64.  ``dense=False`` (large tables):
    only the selected rows are read and returned, as (y, (their ids ascending, their new values),
    the lookup dict).
    """
    sel = lookup(cfg, decode(q, cfg.dtype), decode(C, cfg.dtype), decode(Cp, cfg.dtype), score="idw")
    y = round_to_storage(gather_sum(sel["rows"], sel["w"], V, cfg.dtype), cfg.dtype)
    e = round_to_storage(y - decode(target, cfg.dtype), cfg.dtype)
    uniq = np.unique(sel["rows"])
    g = value_grad_rows(sel["rows"], sel["w"], e, F64, uniq)
    new_rows = round_to_storage(decode(V[uniq], cfg.dtype) - lr * g, cfg.dtype)
    if not dense:
        return y, (uniq, new_rows), sel
    Vn = decode(V, cfg.dtype).copy()
    Vn[uniq] = new_rows
    return y, Vn, sel


def diagnostics(rows: np.ndarray, w: np.ndarray, n_keys: int, n_keys2: int):
    """Monitoring signals of one batch's selection ``rows`` [T, h, k] with weights ``w``.

    ([Blog] §11.2: the codebook hit distribution, each sub-key's hit count and
    the candidate softmax entropy are the signals to watch; §9.3: per-sub-key
    hit counts and gradient density; [PKM-summary] key results: memory usage,
    the share of slots in use, rises above 80% with BatchNorm.)  Returns
    ``hits_c`` [h, |C|] and ``hits_cp`` [h, |C'|]: how many selected slots of
    head h use sub-key i of C (row // |C'| == i) or j of C' (row % |C'| == j);
    ``used`` [1 + h]: distinct rows selected over all heads, then per head;
    ``entropy`` [T, h]: -sum_s w log w (terms with w = 0 count 0), float64.
    """
    T, h, k = rows.shape
    hits_c = np.zeros((h, n_keys), dtype=np.int64)
    hits_cp = np.zeros((h, n_keys2), dtype=np.int64)
    used = np.zeros(1 + h, dtype=np.int64)
    for hh in range(h):
        r = rows[:, hh, :].reshape(-1).astype(np.int64)
        hits_c[hh] = np.bincount(r // n_keys2, minlength=n_keys)
        hits_cp[hh] = np.bincount(r % n_keys2, minlength=n_keys2)
        used[1 + hh] = np.unique(r).size
    used[0] = np.unique(rows).size
    wf = np.asarray(w, dtype=np.float64)
    with np.errstate(divide="ignore", invalid="ignore"):
        terms = np.where(wf > 0, -wf * np.log(np.where(wf > 0, wf, 1.0)), 0.0)
    return hits_c, hits_cp, used, terms.sum(axis=-1)


def weight_grad(rows: np.ndarray, dY: np.ndarray, V: np.ndarray, dtype: str, chunk: int = 256) -> np.ndarray:
    """dw[t,h,s] = <dY[t], V[rows[t,h,s]]> (y is linear in each weight)."""
    T = rows.shape[0]
    dw = np.zeros(rows.shape, dtype=np.float64)
    for lo in range(0, T, chunk):
        hi = min(T, lo + chunk)
        r = rows[lo:hi].reshape(hi - lo, -1)
        vv = decode(V[r.reshape(-1)], dtype).reshape(hi - lo, r.shape[1], -1)
        dy = decode(dY[lo:hi], dtype)
        dw[lo:hi] = np.einsum("tsd,td->ts", vv, dy).reshape(dw[lo:hi].shape)
    return dw


def softmax_backward(w: np.ndarray, dw: np.ndarray, tau: float) -> np.ndarray:
    """Gradient w.r.t. the selected scores: ds = w * (dw - sum_s w dw) / tau."""
    return w * (dw - (w * dw).sum(axis=-1, keepdims=True)) / tau


def subkey_backward(cfg, rows: np.ndarray, ds: np.ndarray, q: np.ndarray, C: np.ndarray, Cp: np.ndarray):
    """Gradients through the selected sub-keys only ([Blog] §9.2).

    Score of selection s: q1.C[i_s] + q2.C'[j_s] with i_s = row // |C'| and
    j_s = row % |C'|; the top-k choices themselves carry no gradient.
    Returns dq [T, h*dq], dC, dC'.
    """
    T, h, k = rows.shape
    half = cfg.dq // 2
    i_all = rows // cfg.n_keys2
    j_all = rows % cfg.n_keys2
    q1_all, q2_all = split_heads(q, h, cfg.dq)
    dq = np.zeros((T, h, cfg.dq), dtype=np.float64)
    dC = np.zeros_like(C)
    dCp = np.zeros_like(Cp)
    step = 512
    for lo in range(0, T, step):
        sl = slice(lo, min(T, lo + step))
        i, j, d_s = i_all[sl], j_all[sl], ds[sl]
        hh = np.broadcast_to(np.arange(h)[None, :, None], i.shape)
        dq[sl, :, :half] = np.einsum("ths,thsd->thd", d_s, C[hh, i])
        dq[sl, :, half:] = np.einsum("ths,thsd->thd", d_s, Cp[hh, j])
        np.add.at(dC, (hh.reshape(-1), i.reshape(-1)),
                  (d_s[..., None] * q1_all[sl][:, :, None, :]).reshape(-1, half))
        np.add.at(dCp, (hh.reshape(-1), j.reshape(-1)),
                  (d_s[..., None] * q2_all[sl][:, :, None, :]).reshape(-1, half))
    return dq.reshape(T, h * cfg.dq), dC, dCp


def batchnorm_backward(dq: np.ndarray, xhat: np.ndarray, gamma: np.ndarray, var: np.ndarray, eps: float):
    """Backward of batch-statistics BatchNorm: returns dq_pre, dgamma, dbeta.

    With q = gamma*xhat + beta and xhat = (q_pre - mean)/sqrt(var + eps), mean
    and var being functions of the whole batch:
    dq_pre = gamma/sqrt(var+eps) * (dq - mean_t(dq) - xhat * mean_t(dq*xhat)).
    """
    dbeta = dq.sum(axis=0)
    dgamma = (dq * xhat).sum(axis=0)
    dq_pre = gamma / np.sqrt(var + eps) * (dq - dq.mean(axis=0) - xhat * (dq * xhat).mean(axis=0))
    return dq_pre, dgamma, dbeta


def backward(cfg, inp: dict, fwd: dict, dY: np.ndarray, dv_rows=None, dense_dv: bool = False):
    """Gradients of sum(dY * m(x)) for a forward ``fwd`` computed over all tokens.

    Returns dw, ds, dq, dq_pre, dC, dCp, dWq, dgamma, dbeta, dx, and dV either
    dense (``dense_dv``) or for the rows in ``dv_rows``.
    """
    assert len(fwd["tokens"]) == cfg.T, "backward needs the forward of every token"
    rows, w = fwd["rows"], fwd["w"]
    dw = weight_grad(rows, dY, inp["V"], cfg.dtype)
    ds = softmax_backward(w, dw, cfg.temperature)
    C = decode(inp["C"], cfg.dtype)
    Cp = decode(inp["Cp"], cfg.dtype)
    dq, dC, dCp = subkey_backward(cfg, rows, ds, fwd["q"], C, Cp)
    if cfg.bn:
        dq_pre, dgamma, dbeta = batchnorm_backward(dq, fwd["xhat"], inp["gamma"].astype(np.float64),
                                                   fwd["var"], cfg.bn_eps)
    else:
        dq_pre, dgamma, dbeta = dq, None, None
    x = decode(inp["x"], cfg.dtype)
    Wq = decode(inp["Wq"], cfg.dtype)
    out = {"dw": dw, "ds": ds, "dq": dq, "dq_pre": dq_pre, "dC": dC, "dCp": dCp,
           "dWq": dq_pre.T @ x, "dx": dq_pre @ Wq, "dgamma": dgamma, "dbeta": dbeta,
           "touched": np.unique(rows)}
    if dense_dv:
        out["dV"] = value_grad_dense(rows, w, dY, cfg.dtype, cfg.slots)
    if dv_rows is not None:
        out["dV_rows"] = value_grad_rows(rows, w, dY, cfg.dtype, dv_rows)
    return out
