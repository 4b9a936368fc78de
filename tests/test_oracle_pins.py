"""Pins of the fp64 CPU oracle against facts fixed by the pages and by mathematics.

Nothing here retypes an oracle formula: each check uses an independent route
(brute force over every full key, pure-Python sorting, library routines on
special cases, closed forms, finite differences, conservation identities),
chosen so that a dropped term, a wrong sign or index, or a transposed operand
in the oracle fails at least one test.  CPU only.
"""
import itertools
import json
import math
import os

import numpy as np
import pytest
import scipy.special
import scipy.stats
import torch

import pkm_inputs as pi
from oracle import pkm_oracle as O

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _cfg(**kw):
    base = dict(T=16, d=12, heads=2, dq=8, n_keys=6, n_keys2=5, topk=4, d_value=10,
                dtype="f32", bn=False, seed=11)
    base.update(kw)
    return pi.custom(**base)


# ---------------------------------------------------------------------------
# the pages' printed counts
# ---------------------------------------------------------------------------
def test_page_counts_product_keys_and_candidates():
    g = json.load(open(os.path.join(GOLDEN, "page_counts.json")))
    pk = g["product_of_two_codebooks"]
    n1, n2 = pk["n_keys"], pk["n_keys2"]
    # every (i, j) gets its own row and every row in [0, n1*n2) is reached
    i = np.arange(n1, dtype=np.int64)[:, None]
    j = np.arange(n2, dtype=np.int64)[None, :]
    _, rows = O.candidates(i.reshape(1, -1)[:, :, None].squeeze(-1), np.zeros((1, n1)),
                           j.reshape(1, -1), np.zeros((1, n2)), n2)
    assert rows.size == pk["product_keys"]
    assert np.array_equal(np.sort(rows.reshape(-1)), np.arange(pk["product_keys"]))
    assert n1 + n2 == pk["stored_subkeys"]

    cc = g["candidate_count"]
    sc, rw = O.candidates(np.arange(cc["k1"])[None], np.ones((1, cc["k1"])),
                          np.arange(cc["k2"])[None], np.ones((1, cc["k2"])), 100)
    assert sc.shape[-1] == cc["candidates"] and len(set(rw.reshape(-1).tolist())) == cc["candidates"]

    lg = g["large_codebooks"]
    assert lg["n_keys"] * lg["n_keys2"] == lg["product_keys"]
    ps = g["paper_setting"]
    assert pi.CONFIGS["paper"].slots == ps["slots_large"]
    assert pi.CONFIGS["paper"].heads == ps["heads"] and pi.CONFIGS["paper"].topk == ps["topk"]


# ---------------------------------------------------------------------------
# storage rounding
# ---------------------------------------------------------------------------
def test_round_to_bf16_special_values():
    one = 1.0
    cases = {
        one: one,
        one + 2.0 ** -8: one,                        # tie -> even mantissa (1.0)
        one + 3 * 2.0 ** -8: one + 2.0 ** -6,        # tie -> even mantissa (1 + 2/128)
        one + 2.0 ** -8 + 2.0 ** -30: one + 2.0 ** -7,  # just above the tie
        -(one + 2.0 ** -8): -one,
        0.0: 0.0,
        2.0 ** -130: 2.0 ** -130,                    # subnormal, exactly representable
        3 * 2.0 ** -134: 2.0 ** -132,                # subnormal tie (1.5 * 2^-133) -> even (2 * 2^-133)
    }
    for v, want in cases.items():
        assert O.round_to_bf16(np.array([v]))[0] == want, v


def test_round_to_bf16_matches_torch_cast():
    a = pi.random_array(5, 0, (4096,), std=3.0).astype(np.float32)
    a = np.concatenate([a, a * 1e-30, a * 1e30])
    ref = torch.from_numpy(a).to(torch.bfloat16).to(torch.float64).numpy()
    assert np.array_equal(O.round_to_bf16(a.astype(np.float64)), ref)


# ---------------------------------------------------------------------------
# a1: projection
# ---------------------------------------------------------------------------
def test_project_permutation_and_scaling():
    x = pi.random_array(1, 0, (7, 5)).astype(np.float64)
    perm = np.array([3, 0, 4, 1, 2])
    W = np.zeros((5, 5))
    W[np.arange(5), perm] = np.array([1.0, 2.0, -1.0, 0.5, 3.0])   # output f reads input perm[f]
    q = O.project(x, W)
    assert np.array_equal(q, x[:, perm] * np.array([1.0, 2.0, -1.0, 0.5, 3.0]))
    # rectangular: 3 outputs from 5 inputs; output f = sum of inputs f and f+2
    W2 = np.zeros((3, 5))
    for f in range(3):
        W2[f, f] = W2[f, f + 2] = 1.0
    assert np.array_equal(O.project(x, W2), x[:, 0:3] + x[:, 2:5])


# ---------------------------------------------------------------------------
# a2: BatchNorm
# ---------------------------------------------------------------------------
def test_batchnorm_closed_form_and_torch():
    qp = pi.random_array(2, 0, (257, 9), std=4.0).astype(np.float64) + 3.0
    eps = 1e-5
    g = np.linspace(0.5, 2.0, 9)
    b = np.linspace(-1.0, 1.0, 9)
    q, mean, var, xhat = O.batchnorm_forward(qp, g, b, eps)
    # batch mean of the output is beta, biased variance is gamma^2 var/(var+eps)
    np.testing.assert_allclose(q.mean(0), b, atol=1e-12)
    np.testing.assert_allclose(((q - q.mean(0)) ** 2).mean(0), g ** 2 * var / (var + eps), rtol=1e-12)
    ref = torch.nn.functional.batch_norm(torch.from_numpy(qp), None, None, torch.from_numpy(g),
                                         torch.from_numpy(b), training=True, eps=eps).numpy()
    np.testing.assert_allclose(q, ref, rtol=1e-12, atol=1e-12)
    # two tokens a, b: xhat = +-(a-b)/2 / sqrt((a-b)^2/4 + eps)
    two = np.array([[3.0], [1.0]])
    _, _, _, xh = O.batchnorm_forward(two, np.ones(1), np.zeros(1), eps)
    assert math.isclose(xh[0, 0], 1.0 / math.sqrt(1.0 + eps), rel_tol=1e-15)
    assert math.isclose(xh[1, 0], -1.0 / math.sqrt(1.0 + eps), rel_tol=1e-15)


# ---------------------------------------------------------------------------
# a3: sub-key scores
# ---------------------------------------------------------------------------
def test_subkey_scores_identity_codebooks():
    T, h, dq = 5, 3, 8
    half = dq // 2
    q = pi.random_array(3, 0, (T, h * dq)).astype(np.float64)
    C = np.stack([np.eye(half) * (hh + 1) for hh in range(h)])          # C[h, i] = (h+1) e_i
    Cp = np.stack([-np.eye(half)[::-1] for _ in range(h)])              # C'[h, j] = -e_{half-1-j}
    q1, q2 = O.split_heads(q, h, dq)
    s1, s2 = O.subkey_scores(q1, q2, C, Cp)
    qh = q.reshape(T, h, dq)
    for hh in range(h):
        np.testing.assert_array_equal(s1[:, hh, :], qh[:, hh, :half] * (hh + 1))
        np.testing.assert_array_equal(s2[:, hh, :], -qh[:, hh, half:][:, ::-1])


# ---------------------------------------------------------------------------
# a4: per-half top-k
# ---------------------------------------------------------------------------
def test_topk_sorted_against_python_sort():
    rng = np.random.Generator(np.random.PCG64(7))
    for trial in range(200):
        n = int(rng.integers(1, 40))
        k = int(rng.integers(1, n + 1))
        s = rng.integers(-3, 4, size=n).astype(np.float64) * (0.5 if trial % 2 else 1.0)
        if trial % 5 == 0:
            s[s == 0] = -0.0           # -0 ties with +0
            s[:2] = 0.0
        idx, val = O.topk_sorted(s[None], k)
        want = sorted(range(n), key=lambda i: (-float(s[i]) + 0.0, i))[:k]
        assert idx[0].tolist() == want
        assert val[0].tolist() == [s[i] for i in want]


# ---------------------------------------------------------------------------
# a4 + a5: product-key selection is the exact top-k of the full key set
# ---------------------------------------------------------------------------
def _python_brute(q, C, Cp, k):
    """Pure-Python loops over every (i, j): score of [C[h,i]; C'[h,j]] and row i*|C'|+j."""
    T = q.shape[0]
    h, nk, half = C.shape
    nk2 = Cp.shape[1]
    rows = np.zeros((T, h, k), dtype=np.int64)
    for t in range(T):
        for hh in range(h):
            qv = q[t, hh * 2 * half:(hh + 1) * 2 * half]
            cand = []
            for i in range(nk):
                for j in range(nk2):
                    key = list(C[hh, i]) + list(Cp[hh, j])
                    sc = sum(float(a) * float(b) for a, b in zip(qv, key))
                    cand.append((-sc, i * nk2 + j))
            cand.sort()
            rows[t, hh] = [r for _, r in cand[:k]]
    return rows


def test_brute_force_matches_python_loops_integer_ties():
    cfg = _cfg(T=6, heads=2, dq=4, n_keys=4, n_keys2=3, topk=5, x_kind="int", wq_kind="int",
               key_kind="int", int_range=1)
    inp = pi.make_inputs(cfg)
    q = O.query(cfg, inp)["q"]
    C, Cp = O.decode(inp["C"], "f32"), O.decode(inp["Cp"], "f32")
    rows, _ = O.brute_force_select(cfg, q, C, Cp)
    assert np.array_equal(rows, _python_brute(q, C, Cp, cfg.topk))


@pytest.mark.parametrize("seed", range(40))
def test_product_key_selection_is_exact_topk(seed):
    rng = np.random.Generator(np.random.PCG64(1000 + seed))
    nk = int(rng.integers(1, 17))
    nk2 = int(rng.integers(1, 17))
    if seed % 4 == 0:
        nk2 = nk
    k = int(rng.integers(1, min(nk, nk2) + 1))
    if seed % 4 == 0:
        k = nk                      # k = |C| = |C'|: the candidate set is every key
    h = int(rng.integers(1, 4))
    dq = int(rng.choice([2, 6, 32]))
    integer = seed % 2 == 1
    cfg = _cfg(T=int(rng.integers(1, 9)), d=int(rng.integers(1, 9)), heads=h, dq=dq, n_keys=nk,
               n_keys2=nk2, topk=k, seed=seed, bn=(seed % 3 == 0) and not integer,
               **({"x_kind": "int", "wq_kind": "int", "key_kind": "int", "int_range": 1} if integer else {}))
    inp = pi.make_inputs(cfg)
    fwd = O.forward(cfg, inp)
    C, Cp = O.decode(inp["C"], "f32"), O.decode(inp["Cp"], "f32")
    rows, scores = O.brute_force_select(cfg, fwd["q"], C, Cp)
    if integer:
        assert np.array_equal(fwd["rows"], rows)            # exact, ties by lowest row
        assert np.array_equal(fwd["scores"], scores)
    else:
        np.testing.assert_allclose(fwd["scores"], scores, rtol=1e-12, atol=1e-12)
        assert np.array_equal(fwd["rows"], rows)
    if seed % 4 == 0:
        assert fwd["sub_idx1"].shape[-1] == nk              # every sub-key is a candidate


def _topk1_case(seed):
    """A random tiny shape (as in test_product_key_selection_is_exact_topk) and its forward."""
    rng = np.random.Generator(np.random.PCG64(2000 + seed))
    nk = int(rng.integers(1, 17))
    nk2 = int(rng.integers(1, 17))
    k = int(rng.integers(1, min(nk, nk2) + 1))
    if seed % 5 == 0:
        k = min(nk, nk2)            # k + 1 exceeds one half's codebook
    integer = seed % 2 == 1
    cfg = _cfg(T=int(rng.integers(1, 9)), d=int(rng.integers(1, 9)), heads=int(rng.integers(1, 4)),
               dq=int(rng.choice([2, 6, 32])), n_keys=nk, n_keys2=nk2, topk=k, seed=seed,
               bn=(seed % 3 == 0) and not integer,
               **({"x_kind": "int", "wq_kind": "int", "key_kind": "int", "int_range": 1} if integer else {}))
    return cfg, integer


@pytest.mark.parametrize("seed", range(40))
def test_top_k_plus_one_list_is_exact(seed):
    # the (k+1)-best full keys that decide the near-tie rule are the exact top-(k+1) of the full key set
    cfg, integer = _topk1_case(seed)
    inp = pi.make_inputs(cfg)
    fwd = O.forward(cfg, inp)
    C, Cp = O.decode(inp["C"], "f32"), O.decode(inp["Cp"], "f32")
    kk = min(cfg.topk + 1, cfg.slots)
    rows, scores = O.brute_force_select(pi.custom(**{**cfg.__dict__, "topk": kk}), fwd["q"], C, Cp)
    assert fwd["rows_k1"].shape[-1] == kk
    assert np.array_equal(fwd["rows_k1"], rows)
    if integer:
        assert np.array_equal(fwd["scores_k1"], scores)
    else:
        np.testing.assert_allclose(fwd["scores_k1"], scores, rtol=1e-12, atol=1e-12)
    # its first k entries are the selection itself
    assert np.array_equal(fwd["rows_k1"][..., :cfg.topk], fwd["rows"])


def test_selection_integer_ties_small_brute():
    cfg = _cfg(T=8, heads=3, dq=6, n_keys=5, n_keys2=7, topk=6, x_kind="int", wq_kind="int",
               key_kind="int", int_range=1, seed=5)
    inp = pi.make_inputs(cfg)
    fwd = O.forward(cfg, inp)
    C, Cp = O.decode(inp["C"], "f32"), O.decode(inp["Cp"], "f32")
    assert np.array_equal(fwd["rows"], _python_brute(fwd["q"], C, Cp, cfg.topk))
    # the data really has ties among selected scores
    assert any(len(set(r.tolist())) < len(r) for r in fwd["scores"].reshape(-1, cfg.topk))


# ---------------------------------------------------------------------------
# a5: softmax
# ---------------------------------------------------------------------------
def test_softmax_closed_forms():
    s = pi.random_array(4, 0, (50, 3, 9), std=5.0).astype(np.float64)
    s = -np.sort(-s, axis=-1)
    for tau in (1.0, 0.37, 4.0):
        w = O.softmax(s, tau)
        np.testing.assert_allclose(w.sum(-1), 1.0, atol=1e-14)
        np.testing.assert_allclose(np.log(w[..., 0] / w[..., 3]), (s[..., 0] - s[..., 3]) / tau, rtol=1e-10)
        np.testing.assert_allclose(w, scipy.special.softmax(s / tau, axis=-1), rtol=1e-13)
        assert np.all(np.diff(w, axis=-1) <= 0)
    assert np.array_equal(O.softmax(s[..., :1], 1.0), np.ones_like(s[..., :1]))


# ---------------------------------------------------------------------------
# a6: gather-sum
# ---------------------------------------------------------------------------
def _dense_A(rows, w, n_rows):
    T = rows.shape[0]
    A = np.zeros((T, n_rows))
    for t in range(T):
        for r, ww in zip(rows[t].reshape(-1), w[t].reshape(-1)):
            A[t, r] += ww
    return A


@pytest.mark.parametrize("dtype", ["f32", "bf16"])
def test_gather_sum_dense_identity(dtype):
    rows, w = pi.random_selection(3, T=40, heads=3, k=5, n_rows=30)
    V = pi.random_array(3, 1, (30, 17), dtype=dtype)
    y = O.gather_sum(rows, w.astype(np.float64), V, dtype, chunk=7)
    Vd = torch.from_numpy(pi.bf16_bits_to_f32(V) if dtype == "bf16" else V).double().numpy()
    np.testing.assert_allclose(y, _dense_A(rows, w.astype(np.float64), 30) @ Vd, rtol=1e-12, atol=1e-14)


def test_gather_k1_is_row_copy_and_heads_add():
    cfg = _cfg(topk=1, heads=1, T=20, d_value=12)
    inp = pi.make_inputs(cfg)
    f = O.forward(cfg, inp)
    np.testing.assert_array_equal(f["w"], 1.0)
    np.testing.assert_array_equal(f["y"], O.decode(inp["V"], "f32")[f["rows"][:, 0, 0]])
    # h heads = sum of single-head memories built from each head's slice (BN is per feature)
    cfg3 = _cfg(heads=3, bn=True, T=24)
    inp3 = pi.make_inputs(cfg3)
    y3 = O.forward(cfg3, inp3)["y"]
    acc = np.zeros_like(y3)
    for hh in range(3):
        c1 = pi.custom(**{**cfg3.__dict__, "heads": 1})
        sl = slice(hh * cfg3.dq, (hh + 1) * cfg3.dq)
        inp1 = dict(inp3, Wq=inp3["Wq"][sl], C=inp3["C"][hh:hh + 1], Cp=inp3["Cp"][hh:hh + 1],
                    gamma=inp3["gamma"][sl], beta=inp3["beta"][sl])
        acc += O.forward(c1, inp1)["y"]
    np.testing.assert_allclose(y3, acc, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# a8: sparse value gradient
# ---------------------------------------------------------------------------
def test_value_grad_dense_identity_and_conservation():
    rows, w = pi.random_selection(9, T=33, heads=2, k=6, n_rows=25)
    w = w.astype(np.float64)
    w /= w.sum(-1, keepdims=True)                 # exactly normalised in float64
    dY = pi.random_array(9, 2, (33, 11))
    dV = O.value_grad_dense(rows, w.astype(np.float64), dY, "f32", 25)
    A = _dense_A(rows, w.astype(np.float64), 25)
    np.testing.assert_allclose(dV, A.T @ dY.astype(np.float64), rtol=1e-12, atol=1e-13)
    # weights of each head sum to 1: sum over rows of dV = heads * sum over tokens of dY
    np.testing.assert_allclose(dV.sum(0), 2 * dY.astype(np.float64).sum(0), rtol=1e-10)
    # untouched rows are exactly zero; the by-row routine agrees with the dense one
    untouched = np.setdiff1d(np.arange(25), rows)
    assert np.all(dV[untouched] == 0)
    which = np.array([0, 3, 24, 7, 7])
    np.testing.assert_allclose(O.value_grad_rows(rows, w.astype(np.float64), dY, "f32", which),
                               dV[which], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# a7, a9, a10: finite differences of every gradient, exact (f64) arithmetic
# ---------------------------------------------------------------------------
def _loss_and_rows(cfg, inp, dY):
    f = O.forward(cfg, inp)
    return float((dY * f["y"]).sum()), f["rows"]


@pytest.mark.parametrize("bn,tau", [(False, 1.0), (True, 1.0), (False, 0.37), (True, 0.37)])
def test_gradients_by_finite_differences(bn, tau):
    # tau != 1 pins the softmax backward's 1/tau (the loss is differentiated through softmax(s/tau))
    cfg = _cfg(T=12, d=7, heads=2, dq=6, n_keys=5, n_keys2=4, topk=3, d_value=5, dtype="f64",
               bn=bn, seed=21, temperature=tau)
    raw = pi.make_inputs(cfg)
    inp = {k: (v.astype(np.float64) if isinstance(v, np.ndarray) and v.dtype == np.float32 else v)
           for k, v in raw.items()}
    inp["gamma"] = np.linspace(0.8, 1.3, cfg.F)
    inp["beta"] = np.linspace(-0.2, 0.3, cfg.F)
    dY = pi.random_array(21, 7, (cfg.T, cfg.d_value)).astype(np.float64)
    fwd = O.forward(cfg, inp)
    g = O.backward(cfg, inp, fwd, dY, dense_dv=True)
    base_rows = fwd["rows"]
    grads = {"x": g["dx"], "Wq": g["dWq"], "C": g["dC"], "Cp": g["dCp"], "V": g["dV"]}
    if bn:
        grads["gamma"], grads["beta"] = g["dgamma"], g["dbeta"]
    eps = 1e-6
    rng = np.random.Generator(np.random.PCG64(5))
    checked = 0
    for name, G in grads.items():
        flat_n = inp[name].size
        picks = list(rng.choice(flat_n, size=min(flat_n, 12), replace=False))
        nz = np.flatnonzero(G.reshape(-1))
        picks += list(rng.choice(nz, size=min(len(nz), 12), replace=False)) if len(nz) else []
        for p in picks:
            vals = []
            for sgn in (+1, -1):
                pert = dict(inp)
                a = inp[name].copy().reshape(-1)
                a[p] += sgn * eps
                pert[name] = a.reshape(inp[name].shape)
                L, rows = _loss_and_rows(cfg, pert, dY)
                vals.append((L, rows))
            if not (np.array_equal(vals[0][1], base_rows) and np.array_equal(vals[1][1], base_rows)):
                continue                # the selection moved: the loss is not differentiable here
            fd = (vals[0][0] - vals[1][0]) / (2 * eps)
            an = G.reshape(-1)[p]
            assert abs(fd - an) <= 1e-6 * max(1.0, abs(an)), (name, p, fd, an)
            checked += 1
    assert checked > 60


def test_backward_invariants():
    cfg = _cfg(T=40, d=9, heads=2, dq=8, n_keys=7, n_keys2=6, topk=4, d_value=6, bn=True, seed=8)
    inp = pi.make_inputs(cfg, with_dy=True)
    fwd = O.forward(cfg, inp)
    g = O.backward(cfg, inp, fwd, inp["dY"], dense_dv=True)
    np.testing.assert_allclose(g["ds"].sum(-1), 0.0, atol=1e-13)            # softmax backward
    np.testing.assert_allclose(g["dq_pre"].sum(0), 0.0, atol=1e-11)         # BN: mean removed
    # sum_t xhat^2 = T var/(var+eps), hence sum_t dq_pre*xhat = rstd*eps/(var+eps) * sum_t dq*xhat (gamma = 1)
    var = fwd["var"]
    rstd = 1.0 / np.sqrt(var + cfg.bn_eps)
    np.testing.assert_allclose((g["dq_pre"] * fwd["xhat"]).sum(0),
                               rstd * cfg.bn_eps / (var + cfg.bn_eps) * (g["dq"] * fwd["xhat"]).sum(0),
                               rtol=1e-8, atol=1e-13)
    np.testing.assert_allclose(g["dV"].sum(0), cfg.heads * inp["dY"].astype(np.float64).sum(0), rtol=1e-10)
    assert np.array_equal(g["touched"], np.flatnonzero(np.abs(g["dV"]).sum(1) > 0))
    # dC only on sub-keys that appear in a final selection
    used1 = np.zeros((cfg.heads, cfg.n_keys), bool)
    for t, hh, s in itertools.product(range(cfg.T), range(cfg.heads), range(cfg.topk)):
        used1[hh, fwd["rows"][t, hh, s] // cfg.n_keys2] = True
    assert np.all(g["dC"][~used1] == 0)


def test_value_grad_rows_sampled_matches_dense_on_small_workload_shape():
    rows, w = pi.random_selection(12, T=256, heads=4, k=32, n_rows=4096, zipf=1.0)
    dY = pi.random_array(12, 3, (256, 24), dtype="bf16")
    dense = O.value_grad_dense(rows, w.astype(np.float64), dY, "bf16", 4096)
    which = np.unique(rows)[::37]
    np.testing.assert_allclose(O.value_grad_rows(rows, w.astype(np.float64), dY, "bf16", which),
                               dense[which], rtol=1e-12, atol=1e-13)


# ---------------------------------------------------------------------------
# Sparse Adam on the touched value rows ([Blog] §6.3)
# ---------------------------------------------------------------------------

def _adam_iterate(V0, steps, lr, b1, b2, eps):
    """Run O.sparse_adam_rows over ``steps`` = [(rows, grad_rows)], carrying the dense state."""
    V = V0.copy()
    m = np.zeros_like(V)
    v = np.zeros_like(V)
    for n, (rows, g) in enumerate(steps, start=1):
        V[rows], m[rows], v[rows] = O.sparse_adam_rows(V[rows], m[rows], v[rows], g, lr, b1, b2, eps, n, O.F64)
    return V, m, v


def test_sparse_adam_all_rows_touched_matches_dense_adam():
    # every row gets gradient at every step: lazy Adam and torch's dense Adam coincide
    rng = np.random.default_rng(5)
    V0 = rng.standard_normal((6, 5))
    grads = [rng.standard_normal((6, 5)) * (0.1 + n) for n in range(5)]
    lr, b1, b2, eps = 1e-2, 0.9, 0.999, 1e-8
    V, m, v = _adam_iterate(V0, [(np.arange(6), g) for g in grads], lr, b1, b2, eps)
    p = torch.nn.Parameter(torch.tensor(V0))
    opt = torch.optim.Adam([p], lr=lr, betas=(b1, b2), eps=eps)
    for g in grads:
        p.grad = torch.tensor(g)
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(V, p.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m, st["exp_avg"].numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(v, st["exp_avg_sq"].numpy(), rtol=1e-12, atol=1e-14)


def test_sparse_adam_lazy_rows_match_torch_sparse_adam():
    # rows without gradient keep value and moments; bias correction counts global
    # steps.  torch's SparseAdam adds eps before its bias correction, so with a
    # negligible eps (it rejects 0) the two forms agree to rounding.
    rng = np.random.default_rng(6)
    n_rows, d = 40, 3
    V0 = rng.standard_normal((n_rows, d))
    steps = []
    for n in range(6):
        rows = np.sort(rng.choice(n_rows, size=rng.integers(1, n_rows), replace=False))
        steps.append((rows, rng.standard_normal((rows.size, d))))
    lr, b1, b2 = 3e-2, 0.8, 0.95
    V, m, v = _adam_iterate(V0, steps, lr, b1, b2, 1e-30)
    p = torch.nn.Parameter(torch.tensor(V0))
    opt = torch.optim.SparseAdam([p], lr=lr, betas=(b1, b2), eps=1e-30)
    for rows, g in steps:
        p.grad = torch.sparse_coo_tensor(torch.tensor(rows)[None], torch.tensor(g), (n_rows, d))
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(V, p.detach().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(m, st["exp_avg"].to_dense().numpy(), rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(v, st["exp_avg_sq"].to_dense().numpy(), rtol=1e-12, atol=1e-14)
    untouched = np.setdiff1d(np.arange(n_rows), np.concatenate([r for r, _ in steps]))
    np.testing.assert_array_equal(V[untouched], V0[untouched])


def test_sparse_adam_first_step_closed_form_and_bf16_rounding():
    # from zero moments the first step moves each element by lr * g / (|g| + eps)
    rng = np.random.default_rng(7)
    g = rng.standard_normal((4, 9))
    g[0, 0] = 0.0
    V0 = rng.standard_normal((4, 9))
    lr, eps = 1e-3, 1e-6
    V1, m1, v1 = O.sparse_adam_rows(V0, np.zeros_like(g), np.zeros_like(g), g, lr, 0.9, 0.999, eps, 1, O.F64)
    np.testing.assert_allclose(V1, V0 - lr * g / (np.abs(g) + eps), rtol=1e-13, atol=1e-16)
    np.testing.assert_allclose(m1, 0.1 * g, rtol=1e-15)
    np.testing.assert_allclose(v1, 0.001 * g * g, rtol=1e-14)
    assert V1[0, 0] == V0[0, 0]
    # bf16 storage: the stored value is the nearest bf16 of the exact update (torch's cast)
    Vb = torch.tensor(V0, dtype=torch.float32).to(torch.bfloat16)
    bits = Vb.view(torch.int16).numpy().view(np.uint16)
    Vb1, _, _ = O.sparse_adam_rows(bits, np.zeros_like(g), np.zeros_like(g), g, lr, 0.9, 0.999, eps, 1, O.BF16)
    exact = Vb.double().numpy() - lr * g / (np.abs(g) + eps)
    want = torch.tensor(exact).to(torch.bfloat16).double().numpy()
    np.testing.assert_array_equal(Vb1, want)



def _adam_rows_iterate(V0, steps, lr, b1, b2, eps, capacity, pool_fill=7.0):
    # the pool starts with stale values: a row's first step must not read them
    n_rows, d = V0.shape
    V = V0.copy()
    slot = -np.ones(n_rows, dtype=np.int64)
    M = np.full((capacity, d), pool_fill)
    Vm = np.full((capacity, d), pool_fill)
    n_used, stepped_all = 0, []
    for t, (rows, g) in enumerate(steps, 1):
        out, slot, M, Vm, n_used, stepped = O.adam_rows_state_step(rows, slot, M, Vm, n_used, capacity, V[rows], g,
                                                                   lr, b1, b2, eps, t, O.F64)
        V[rows] = out
        stepped_all.append(stepped)
    return V, slot, M, Vm, n_used, stepped_all


def test_adam_rows_state_matches_torch_sparse_adam():
    # moments held in slots handed out on a row's first gradient: the same
    # trajectory as torch's SparseAdam (dense state), whatever the pool held
    rng = np.random.default_rng(16)
    n_rows, d = 40, 3
    V0 = rng.standard_normal((n_rows, d))
    steps = []
    for n in range(6):
        rows = np.sort(rng.choice(n_rows, size=rng.integers(1, 25), replace=False))
        steps.append((rows, rng.standard_normal((rows.size, d))))
    lr, b1, b2 = 3e-2, 0.8, 0.95
    V, slot, M, Vm, n_used, _ = _adam_rows_iterate(V0, steps, lr, b1, b2, 1e-30, capacity=n_rows)
    p = torch.nn.Parameter(torch.tensor(V0))
    opt = torch.optim.SparseAdam([p], lr=lr, betas=(b1, b2), eps=1e-30)
    for rows, g in steps:
        p.grad = torch.sparse_coo_tensor(torch.tensor(rows)[None], torch.tensor(g), (n_rows, d))
        opt.step()
    st = opt.state[p]
    np.testing.assert_allclose(V, p.detach().numpy(), rtol=1e-12, atol=1e-14)
    seen = np.unique(np.concatenate([r for r, _ in steps]))
    assert n_used == seen.size and sorted(slot[seen]) == list(range(seen.size))
    assert (slot[np.setdiff1d(np.arange(n_rows), seen)] == -1).all()
    np.testing.assert_allclose(M[slot[seen]], st["exp_avg"].to_dense().numpy()[seen], rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(Vm[slot[seen]], st["exp_avg_sq"].to_dense().numpy()[seen], rtol=1e-12, atol=1e-14)


def test_adam_rows_state_slot_rule_worked_example():
    # 10 rows, a pool of 4 slots; slots go to new rows in ascending row order,
    # a row that finds the pool full keeps no state and is not stepped
    V0 = np.arange(20, dtype=np.float64).reshape(10, 2)
    steps = [(np.array([2, 5, 7]), np.ones((3, 2))),
             (np.array([1, 5, 9]), np.ones((3, 2))),
             (np.array([0, 9]), np.ones((2, 2)))]
    V, slot, _, _, n_used, stepped = _adam_rows_iterate(V0, steps, 0.1, 0.9, 0.999, 1e-8, capacity=4)
    assert list(slot) == [-1, 3, 0, -1, -1, 1, -1, 2, -1, -1]
    assert n_used == 7                     # 3 + 2 + 2 rows asked for a slot, 2 of them in vain
    assert [list(x) for x in stepped] == [[True, True, True], [True, True, False], [False, False]]
    np.testing.assert_array_equal(V[[0, 3, 4, 6, 8, 9]], V0[[0, 3, 4, 6, 8, 9]])
    # a first step from zero moments moves each element by lr * g / (|g| + eps)
    np.testing.assert_allclose(V[[2, 7]], V0[[2, 7]] - 0.1 / (1 + 1e-8), rtol=1e-15)


# ---------------------------------------------------------------------------
# Monitoring signals ([Blog] §9.3, §11.2; [PKM-summary] key results)
# ---------------------------------------------------------------------------

def test_diagnostics_against_python_loops():
    rng = np.random.default_rng(8)
    T, h, k, nk, nk2 = 13, 3, 4, 5, 7
    rows = rng.integers(0, nk * nk2, size=(T, h, k)).astype(np.int32)
    w = rng.random((T, h, k))
    w /= w.sum(-1, keepdims=True)
    hc, hcp, used, ent = O.diagnostics(rows, w, nk, nk2)
    for hh in range(h):
        for i in range(nk):
            assert hc[hh, i] == sum(1 for t in range(T) for s in range(k) if rows[t, hh, s] // nk2 == i)
        for j in range(nk2):
            assert hcp[hh, j] == sum(1 for t in range(T) for s in range(k) if rows[t, hh, s] % nk2 == j)
        assert used[1 + hh] == len({int(rows[t, hh, s]) for t in range(T) for s in range(k)})
    assert used[0] == len({int(r) for r in rows.reshape(-1)})
    assert (hc.sum(1) == T * k).all() and (hcp.sum(1) == T * k).all()
    for t in range(T):
        for hh in range(h):
            want = -sum(float(x) * math.log(float(x)) for x in w[t, hh])
            assert abs(ent[t, hh] - want) <= 1e-13


def test_diagnostics_entropy_closed_forms():
    k = 8
    rows = np.arange(3 * 2 * k, dtype=np.int32).reshape(3, 2, k)
    w = np.zeros((3, 2, k))
    w[0] = 1.0 / k                       # uniform: log k
    w[1, :, 0] = 1.0                     # one-hot: 0 (w = 0 terms count 0)
    w[2] = scipy.special.softmax(np.arange(k, dtype=np.float64))
    _, _, used, ent = O.diagnostics(rows, w, 8, 8)
    np.testing.assert_allclose(ent[0], math.log(k), rtol=1e-15)
    assert (ent[1] == 0.0).all()
    np.testing.assert_allclose(ent[2], scipy.stats.entropy(w[2, 0]), rtol=1e-13)
    assert used[0] == 3 * 2 * k and (used[1:] == 3 * k).all()


# ---------------------------------------------------------------------------
# fp8 value storage ([Blog] §16.3)
# ---------------------------------------------------------------------------

def test_e4m3_decode_matches_torch_float8_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = O.e4m3_decode(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).double().numpy()
    assert np.array_equal(np.isnan(ours), np.isnan(ref))
    ok = ~np.isnan(ref)
    np.testing.assert_array_equal(ours[ok], ref[ok])
    assert O.e4m3_decode(np.array([0x7E]))[0] == 448.0 and O.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9


def test_e4m3_encode_matches_torch_cast_including_ties():
    rng = np.random.default_rng(9)
    codes = np.array([c for c in range(256) if not np.isnan(O.e4m3_decode(np.array([c]))[0])], dtype=np.uint8)
    vals = np.unique(O.e4m3_decode(codes))
    mids = (vals[1:] + vals[:-1]) / 2                              # exact ties: the even code wins
    xs = np.concatenate([vals, mids, rng.uniform(-448, 448, 20000), rng.uniform(-0.02, 0.02, 5000),
                         np.array([0.0, -0.0, 2.0 ** -10, -(2.0 ** -10), 447.99])]).astype(np.float32)
    ours = O.e4m3_encode(xs)
    ref = torch.from_numpy(xs).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    np.testing.assert_array_equal(O.e4m3_decode(ours), O.e4m3_decode(ref))
    # beyond the range the encoder saturates (the row scale keeps quotients inside it)
    assert O.e4m3_decode(O.e4m3_encode(np.array([1e6, -500.0])))[0] == 448.0
    assert O.e4m3_decode(O.e4m3_encode(np.array([1e6, -500.0])))[1] == -448.0


def test_quantize_rows_fp8_closed_forms_and_error_bound():
    rng = np.random.default_rng(10)
    V = rng.standard_normal((50, 64)).astype(np.float32) * np.exp(rng.uniform(-6, 3, (50, 1))).astype(np.float32)
    V[3] = 0.0
    V[4, :] = 0.0
    V[4, 5] = -2.5                                                 # one non-zero element: it maps to -448
    scale, codes = O.quantize_rows_fp8(V, O.F32)
    assert scale[3] == 0 and (codes[3] == 0).all()
    assert codes[4, 5] == 0xFE and (codes[4, np.arange(64) != 5] == 0).all()
    mx = np.abs(V).max(1)
    np.testing.assert_array_equal(scale, (mx / np.float32(448)).astype(np.float32))
    # every row's largest element lands on +-448 (code 0x7E / 0xFE)
    j = np.abs(V).argmax(1)
    r = np.arange(50)[mx > 0]
    assert np.all((codes[r, j[r]] & 0x7F) == 0x7E)
    deq = O.dequantize_rows_fp8(scale, codes)
    # half a unit in the last place of e4m3 (3 mantissa bits) or of its subnormal step, plus fp32 slack
    bound = np.maximum(np.abs(V) * 2.0 ** -4, scale[:, None] * 2.0 ** -10) * (1 + 1e-6) + 1e-30
    assert np.all(np.abs(deq - V) <= bound)


# ---------------------------------------------------------------------------
# FwPKM: IDW scores and the per-chunk memorization write (FwPKM page §2.1-2.2)
# ---------------------------------------------------------------------------

class _Cfg:
    def __init__(self, **kw):
        self.__dict__.update(kw)


def test_idw_scores_closed_forms():
    q1 = np.zeros((1, 1, 2))
    C = np.array([[[3.0, 4.0], [0.0, 0.0], [1.0, 0.0]]])
    s1, _ = O.subkey_scores_idw(q1, q1, C, C)
    np.testing.assert_allclose(s1[0, 0], [-math.log(5.0), -0.5 * math.log(O.IDW_FLOOR), 0.0], rtol=1e-15)


@pytest.mark.parametrize("seed", [0, 1, 2])
def test_idw_product_key_selection_is_exact_topk(seed):
    # the sum of the halves' -log distances is separable, so the product-key search is exact
    rng = np.random.default_rng(40 + seed)
    h, dq, nk, nk2, k, T = 2, 6, 7, 5, 4, 9
    cfg = _Cfg(heads=h, dq=dq, topk=k, n_keys=nk, n_keys2=nk2, temperature=1.0)
    q = rng.standard_normal((T, h * dq))
    C = rng.standard_normal((h, nk, dq // 2))
    Cp = rng.standard_normal((h, nk2, dq // 2))
    sel = O.lookup(cfg, q, C, Cp, score="idw")
    for t in range(T):
        for hh in range(h):
            qa, qb = q[t, hh * dq: hh * dq + dq // 2], q[t, hh * dq + dq // 2: (hh + 1) * dq]
            full = []
            for i in range(nk):
                for j in range(nk2):
                    sc = -math.log(np.linalg.norm(qa - C[hh, i])) - math.log(np.linalg.norm(qb - Cp[hh, j]))
                    full.append((-sc, i * nk2 + j))
            full.sort()
            assert [r for _, r in full[:k]] == list(sel["rows"][t, hh])
            np.testing.assert_allclose(sel["scores"][t, hh], [-v for v, _ in full[:k]], rtol=1e-12)


def test_fwpkm_chunk_write_is_the_gradient_step_of_the_reconstruction_loss():
    rng = np.random.default_rng(41)
    h, dq, nk, k, T, dv, lr = 2, 8, 6, 3, 10, 5, 0.3
    cfg = _Cfg(heads=h, dq=dq, topk=k, n_keys=nk, n_keys2=nk, temperature=1.0, dtype=O.F64)
    q = rng.standard_normal((T, h * dq))
    C = rng.standard_normal((h, nk, dq // 2))
    Cp = rng.standard_normal((h, nk, dq // 2))
    V = rng.standard_normal((nk * nk, dv))
    tgt = rng.standard_normal((T, dv))
    y, Vn, sel = O.fwpkm_chunk(cfg, q, C, Cp, V, tgt, lr)
    # y reads the rows before the write
    np.testing.assert_allclose(y, O.gather_sum(sel["rows"], sel["w"], V, O.F64), rtol=1e-15)

    def loss(Vx):
        yx = O.gather_sum(sel["rows"], sel["w"], Vx, O.F64)
        return 0.5 * ((yx - tgt) ** 2).sum()

    g = (V - Vn) / lr
    eps = 1e-6
    for r in range(nk * nk):
        for c in range(dv):
            E = np.zeros_like(V)
            E[r, c] = eps
            fd = (loss(V + E) - loss(V - E)) / (2 * eps)
            assert abs(fd - g[r, c]) <= 1e-6 * max(1.0, abs(fd))
    untouched = np.setdiff1d(np.arange(nk * nk), np.unique(sel["rows"]))
    np.testing.assert_array_equal(Vn[untouched], V[untouched])


def test_fwpkm_chunk_sparse_output_is_the_dense_table_at_the_selected_rows():
    rng = np.random.default_rng(42)
    h, dq, nk, k, T, dv, lr = 2, 16, 12, 4, 30, 8, 0.7
    cfg = _Cfg(heads=h, dq=dq, topk=k, n_keys=nk, n_keys2=nk, temperature=1.0, dtype=O.BF16)
    q = pi.f32_to_bf16_bits(rng.standard_normal((T, h * dq)).astype(np.float32))
    C = pi.f32_to_bf16_bits(rng.standard_normal((h, nk, dq // 2)).astype(np.float32))
    Cp = pi.f32_to_bf16_bits(rng.standard_normal((h, nk, dq // 2)).astype(np.float32))
    V = pi.f32_to_bf16_bits(rng.standard_normal((nk * nk, dv)).astype(np.float32))
    tgt = pi.f32_to_bf16_bits(rng.standard_normal((T, dv)).astype(np.float32))
    y, Vn, sel = O.fwpkm_chunk(cfg, q, C, Cp, V, tgt, lr)
    y2, (ids, rows_new), sel2 = O.fwpkm_chunk(cfg, q, C, Cp, V, tgt, lr, dense=False)
    np.testing.assert_array_equal(y2, y)
    np.testing.assert_array_equal(ids, np.unique(sel["rows"]))
    np.testing.assert_array_equal(rows_new, Vn[ids])
    assert (Vn[ids] != O.decode(V, O.BF16)[ids]).any()
