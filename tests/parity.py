"""Comparison rules between the HIP path and the CPU oracle (test helpers).

Tolerances (from the stated accuracy targets): fp32 storage 1e-5 relative, bf16
storage 2e-2 relative.  Row outputs (y, dV) compare per row as
max|diff| / max|ref|; reductions (dC, dC', dWq, dgamma, dbeta, dx) compare by
Frobenius norm ratio.

Selections: several answers are correct when scores nearly tie.  A selection G
of one (token, head) is valid iff its k rows are distinct, in range, and

    min_{r in G} s(r) >= max_{r not in G} s(r) - delta,
    delta = 1e-4 * max(|s_(k)|, |s_(k+1)|) + slack,

with s the oracle's fp64 full-key scores (the best row outside G is among the
oracle's k+1 best).  When the k-th / (k+1)-th gap exceeds delta this forces G
to be exactly the oracle's set.  ``slack`` bounds how far the scores can move
when the GPU's bf16 query differs from the oracle's by the allowed one ulp
(zero for fp32 storage and for seeded queries).
"""
from __future__ import annotations

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
