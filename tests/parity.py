"""Comparison rules between the HIP path and the CPU oracle (test helpers).

Tolerances (from the stated accuracy targets): fp32 storage 1e-5 relative, bf16
storage 2e-2 relative.  Row outputs (y, dV) compare per row as
max|diff| / max|ref|; reductions (dC, dC', dWq, dgamma, dbeta, dx) compare by
Frobenius norm ratio.

Selections: several answers are correct when scores nearly tie.  A selection G
of one (token, head) is valid iff its k rows are distinct, in range, and

    min_{r in G} s(r) >= max_{r not in G} s(r) - delta,
    delta = 1e-4 * max(|s_(k)|, |s_(k+1)|) (+ slack),

with s the oracle's fp64 full-key scores (the best row outside G is among the
oracle's k+1 best).  When the k-th / (k+1)-th gap exceeds delta this forces G
to be exactly the oracle's set.  For the dot-product lookup the slack is zero:
with bf16 storage the oracle searches the GPU's own saved bf16 query (the
search input the scores are computed from; the query itself is checked against
the oracle's separately, to one bf16 ulp), so every set outside near ties must
match exactly.  Only the fast-weight IDW scores pass a slack: the fp32 error
bound of their distance formula.

Where a valid selection differs from the oracle's (a near tie), the backward is
compared with the oracle run on that selection (``forced_forward``): its
weights are the oracle's softmax of its own scores of the GPU's rows, so every
gradient has one correct answer and no upstream gradient is masked.
"""
from __future__ import annotations

import os
from concurrent.futures import ThreadPoolExecutor

import numpy as np

TOL = {"f32": 1e-5, "bf16": 2e-2}
REL_GAP = 1e-4


def bf16_bits_to_f64(b):
    return (np.asarray(b).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def to_f64(t) -> np.ndarray:
    """torch tensor (GPU or CPU, fp32 / bf16 / int) -> numpy float64 / int."""
    import torch
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.float().double().numpy()
    if t.is_floating_point():
        return t.double().numpy()
    return t.numpy()


def row_rel_err(a: np.ndarray, ref: np.ndarray) -> np.ndarray:
    a = a.reshape(a.shape[0], -1)
    ref = ref.reshape(ref.shape[0], -1)
    den = np.maximum(np.abs(ref).max(axis=1), 1e-30)
    return np.abs(a - ref).max(axis=1) / den


def fro_rel_err(a: np.ndarray, ref: np.ndarray) -> float:
    den = np.linalg.norm(ref.reshape(-1))
    num = np.linalg.norm((a - ref).reshape(-1))
    return float(num / den) if den > 0 else float(num)


def bf16_ulp(v: np.ndarray) -> np.ndarray:
    _, e = np.frexp(np.asarray(v, dtype=np.float64))
    return np.ldexp(1.0, np.maximum(e - 8, -133))


def q_allowed(q_g: np.ndarray, q_o: np.ndarray) -> np.ndarray:
    """Largest allowed |q_gpu - q_oracle| per element for a bf16 query.

    q is the nearest bf16 of a value the GPU computes in fp32 and the oracle in
    fp64: the two may land on neighbouring bf16 values (one ulp), and where
    q_pre sits near its batch mean the fp32 cancellation error (about 1e-5 of
    the feature's scale) can exceed the ulp of the tiny result.
    """
    scale = np.abs(q_o).max(axis=0, keepdims=True)
    return bf16_ulp(np.maximum(np.abs(q_g), np.abs(q_o))) * 1.0001 + 1e-5 * scale


def full_scores(rows: np.ndarray, s1: np.ndarray, s2: np.ndarray, nk2: int) -> np.ndarray:
    """Oracle score of each row id in rows[n, h, m] from the per-half tables s1[n, h, |C|], s2[n, h, |C'|]."""
    i = rows // nk2
    j = rows % nk2
    return np.take_along_axis(s1, i, axis=-1) + np.take_along_axis(s2, j, axis=-1)


def check_selection(G: np.ndarray, orc_rows_k1: np.ndarray, orc_scores_k1: np.ndarray, score_of,
                    n_rows: int, k: int, slack=None):
    """Validate GPU selections G[n, h, k] (see module doc).

    ``score_of(rows)`` returns the oracle's score of row ids of shape [n, h, m].
    Returns (valid mask, exact-set mask, exact-order mask), each [n, h].
    """
    n, h, _ = G.shape
    in_range = (G >= 0).all(-1) & (G < n_rows).all(-1)
    Gs = np.sort(G, axis=-1)
    distinct = (np.diff(Gs, axis=-1) != 0).all(-1) if k > 1 else np.ones((n, h), bool)
    Gc = np.clip(G, 0, n_rows - 1)
    sG = score_of(Gc)
    kk = orc_rows_k1.shape[-1]
    sk = orc_scores_k1[..., k - 1]
    skp1 = orc_scores_k1[..., k] if kk > k else orc_scores_k1[..., k - 1]
    delta = REL_GAP * np.maximum(np.abs(sk), np.abs(skp1))
    if slack is not None:
        delta = delta + slack
    # best oracle row outside G (among the oracle's k+1 best)
    member = (orc_rows_k1[..., :, None] == G[..., None, :]).any(-1)
    out_scores = np.where(member, -np.inf, orc_scores_k1)
    best_out = out_scores.max(-1)
    valid = in_range & distinct & (sG.min(-1) >= best_out - delta)
    exact_set = (np.sort(orc_rows_k1[..., :k], axis=-1) == Gs).all(-1)
    exact_order = (orc_rows_k1[..., :k] == G).all(-1)
    # order inside G must follow the oracle's scores up to delta
    if k > 1:
        valid &= (np.diff(sG, axis=-1) <= delta[..., None]).all(-1)
    return valid, exact_set, exact_order


def ordered_gaps_exceed(scores: np.ndarray, k: int) -> np.ndarray:
    """[n, h]: every adjacent gap among the oracle's k+1 best exceeds the tie threshold."""
    s = scores[..., : k + 1]
    d = REL_GAP * np.maximum(np.abs(s[..., :-1]), np.abs(s[..., 1:]))
    return ((s[..., :-1] - s[..., 1:]) > d).all(-1)


def lookup_chunks(cfg, q: np.ndarray, C: np.ndarray, Cp: np.ndarray, score: str = "dot", chunk: int = 256) -> dict:
    """The oracle's search (O.lookup, tables kept) for the tokens of ``q``, over token chunks in a thread pool.

    Each token's search is independent of the others, so the chunks' results are concatenated."""
    from oracle import pkm_oracle as O
    n = q.shape[0]
    spans = [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        parts = list(ex.map(lambda sp: O.lookup(cfg, q[sp[0]:sp[1]], C, Cp, keep_tables=True, score=score), spans))
    return {key: (None if parts[0][key] is None else np.concatenate([p[key] for p in parts])) for key in parts[0]}


def judge_selection(cfg, sel: dict, G: np.ndarray, slack=None):
    """Check GPU selections G [n, h, k] against the oracle's search ``sel`` (O.lookup output with tables).

    Asserts: every selection valid (rule above); the exact set wherever the k-th / (k+1)-th gap exceeds
    delta; the exact order wherever every adjacent gap among the k + 1 best exceeds delta.  Returns
    (score_of, exact_set, exact_order); ``score_of(rows)`` gives the oracle's score of row ids [n, h, m]."""
    s1, s2 = sel["s1"], sel["s2"]
    k = cfg.topk

    def score_of(r):
        return full_scores(np.asarray(r).astype(np.int64), s1, s2, cfg.n_keys2)

    valid, exact_set, exact_order = check_selection(G, sel["rows_k1"], sel["scores_k1"], score_of, cfg.slots, k,
                                                    slack)
    assert valid.all(), f"invalid selections at {np.argwhere(~valid)[:5].tolist()}"
    sk = sel["scores_k1"]
    if sk.shape[-1] > k and slack is None:
        gap = (sk[..., k - 1] - sk[..., k]) > REL_GAP * np.maximum(np.abs(sk[..., k - 1]), np.abs(sk[..., k]))
        assert exact_set[gap].all(), f"set differs outside a near tie at {np.argwhere(gap & ~exact_set)[:5].tolist()}"
        ordered = ordered_gaps_exceed(sk, k)
        assert exact_order[ordered].all(), \
            f"order differs outside near ties at {np.argwhere(ordered & ~exact_order)[:5].tolist()}"
    return score_of, exact_set, exact_order


def forced_forward(cfg, ref: dict, sel: dict, q_sel: np.ndarray, G: np.ndarray) -> dict:
    """The oracle's forward state ``ref`` (its own projection and BatchNorm) with the validated GPU selection
    G [T, h, k] in place of its own: rows G, the oracle's scores of them (from ``sel``'s tables, computed on
    the query ``q_sel``), their softmax weights, and q_sel as the query the sub-key gradients read."""
    from oracle import pkm_oracle as O
    s = full_scores(G.astype(np.int64), sel["s1"], sel["s2"], cfg.n_keys2)
    fwd = dict(ref)
    fwd.update(q=q_sel, rows=G.astype(np.int64), scores=s, w=O.softmax(s, cfg.temperature))
    return fwd


def _pool_map(fn, spans):
    with ThreadPoolExecutor(max(1, min(16, os.cpu_count() or 1))) as ex:
        return list(ex.map(fn, spans))


def _spans(n, chunk):
    return [(lo, min(n, lo + chunk)) for lo in range(0, n, chunk)]


def scores_at(cfg, q: np.ndarray, C: np.ndarray, Cp: np.ndarray, G: np.ndarray, chunk: int = 256) -> np.ndarray:
    """The oracle's full-key scores of the rows G [n, h, m] for the queries q [n, h*dq]: its sub-key score
    tables (O.subkey_scores) per token chunk, read at each row's two halves."""
    from oracle import pkm_oracle as O

    def one(sp):
        q1, q2 = O.split_heads(q[sp[0]:sp[1]], cfg.heads, cfg.dq)
        s1, s2 = O.subkey_scores(q1, q2, C, Cp)
        return full_scores(G[sp[0]:sp[1]].astype(np.int64), s1, s2, cfg.n_keys2)
    return np.concatenate(_pool_map(one, _spans(q.shape[0], chunk)))


def backward_chunks(cfg, inp: dict, fwd: dict, dY: np.ndarray, chunk: int = 1024, tokens=None) -> dict:
    """O.backward's outputs (without dV) with its per-token steps (dw, ds, dq and the dC / dC' terms) run
    over token chunks in a thread pool, dC and dC' summed over the chunks; BatchNorm backward, dWq and dx
    as O.backward computes them.  For the full-size tests, where one thread would take minutes.

    ``tokens`` (sorted): run the per-token steps on these tokens only.  Every other token must have a zero
    upstream gradient: its dw, ds and dq are then exactly zero, and so are its dC and dC' terms (the
    BatchNorm backward still spans every token).  ``fwd``'s rows, w and q may then cover ``tokens`` only."""
    from oracle import pkm_oracle as O
    C = O.decode(inp["C"], cfg.dtype)
    Cp = O.decode(inp["Cp"], cfg.dtype)
    if tokens is None:
        tok, rows, w, q = np.arange(cfg.T), fwd["rows"], fwd["w"], fwd["q"]
    else:
        tok = np.asarray(tokens)
        rest = np.setdiff1d(np.arange(cfg.T), tok)
        assert not O.decode(dY[rest], cfg.dtype).any(), "tokens outside ``tokens`` need a zero upstream gradient"
        full = fwd["rows"].shape[0] == cfg.T
        rows, w, q = ((fwd["rows"][tok], fwd["w"][tok], fwd["q"][tok]) if full
                      else (fwd["rows"], fwd["w"], fwd["q"]))
    dYt = dY[tok]

    def one(sp):
        sl = slice(*sp)
        dw = O.weight_grad(rows[sl], dYt[sl], inp["V"], cfg.dtype)
        ds = O.softmax_backward(w[sl], dw, cfg.temperature)
        dq, dC, dCp = O.subkey_backward(cfg, rows[sl], ds, q[sl], C, Cp)
        return dw, ds, dq, dC, dCp
    parts = _pool_map(one, _spans(len(tok), chunk))
    dw = np.zeros((cfg.T,) + rows.shape[1:])
    ds = np.zeros_like(dw)
    dq = np.zeros((cfg.T, cfg.heads * cfg.dq))
    dw[tok] = np.concatenate([p[0] for p in parts])
    ds[tok] = np.concatenate([p[1] for p in parts])
    dq[tok] = np.concatenate([p[2] for p in parts])
    dC = sum(p[3] for p in parts)
    dCp = sum(p[4] for p in parts)
    if cfg.bn:
        dq_pre, dgamma, dbeta = O.batchnorm_backward(dq, fwd["xhat"], inp["gamma"].astype(np.float64), fwd["var"],
                                                     cfg.bn_eps)
    else:
        dq_pre, dgamma, dbeta = dq, None, None
    x = O.decode(inp["x"], cfg.dtype)
    Wq = O.decode(inp["Wq"], cfg.dtype)
    return {"dw": dw, "ds": ds, "dq": dq, "dq_pre": dq_pre, "dC": dC, "dCp": dCp, "dWq": dq_pre.T @ x,
            "dx": dq_pre @ Wq, "dgamma": dgamma, "dbeta": dbeta}
