"""GPU parity of the fast-weight memory (FwPKM) path against the fp64 CPU oracle.

IDW sub-key scores ("Fast-weight Product Key Memory", section 2.2: the negative
log of the Euclidean distance replaces the dot product) through
``pkm_stage_score_topk`` and ``pkm_forward``, and the memorization chunk
(sections 2.1-2.2: read, then a gradient step of the value rows toward the
lookahead targets) through ``pkm_fwpkm_chunk``.

Error model of the selection.  The kernel ranks sub-keys on u = 2 q.c - ||c||^2
(fp32, MFMA accumulation) and reports s = -1/2 log(max(||q||^2 - u, 1e-12)).
Each fp32 sum of n products is off by at most about n * 2^-24 times the sum of
the absolute products, so u is off by at most E = g (2 ||q|| max||c|| +
max||c||^2) with g = (half + 2) 2^-24, and a score near the k-th best (squared
distance d2) by E / (2 d2) (plus the same for ||q||^2).  Two sub-keys whose u
differ by less than 2 E may be ranked either way: ``slack`` turns that into the
score units of the selection rule in tests/parity.py.  On integer inputs every
sum is exact, so indices (lowest first on ties) and the floor of a zero
distance must match exactly.
"""
import numpy as np
import pytest
import torch

import pkm_inputs as pi
from oracle import pkm_oracle as O
from tests import parity as P
from tests.gpu_util import layer_for, note, require_lib, to_dev, upload

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _cfg(**kw):
    base = dict(T=64, d=16, heads=1, dq=32, n_keys=32, n_keys2=32, topk=8, d_value=64, dtype="f32", bn=False,
                seed=3)
    base.update(kw)
    return pi.custom(**base)


def _u_bound(qh: np.ndarray, K: np.ndarray) -> np.ndarray:
    """[n, h]: bound on the fp32 error of u = 2 q.c - ||c||^2 over the sub-keys K [h, m, half]."""
    half = qh.shape[-1]
    g = (half + 2) * 2.0 ** -24
    qn = np.linalg.norm(qh, axis=-1)                  # [n, h]
    cn = np.linalg.norm(K, axis=-1).max(axis=-1)      # [h]
    return g * (2 * qn * cn[None] + cn[None] ** 2 + (qh ** 2).sum(-1))


def _half_slack(qh, K, s_k):
    """Selection slack in score units for a half whose k-th best oracle score is s_k [n, h]."""
    d2 = np.exp(-2.0 * s_k)                           # squared distance of the k-th best
    E = _u_bound(qh, K)
    return 2 * E / np.maximum(d2 - E, 1e-30)


def _score_err(qh, K, top_vals):
    """[n, h]: bound on the fp32 error of any sub-key score among a half's top-k (``top_vals`` [n, h, k])."""
    d2 = np.exp(-2.0 * top_vals[..., 0])
    E = _u_bound(qh, K)
    return E / np.maximum(d2 - E, 1e-30) + 4 * 2.0 ** -24 * np.abs(top_vals).max(-1) + 1e-7


# ---------------------------------------------------------------------------
# a3 + a4 with IDW scores
# ---------------------------------------------------------------------------
IDW_SCORE_CASES = [
    # T, heads, dq, nk, nk2, k, dtype, integer
    (100, 2, 32, 32, 48, 8, "f32", False),
    (257, 4, 256, 256, 256, 32, "f32", False),
    (75, 4, 512, 1024, 1024, 32, "bf16", False),
    (60, 2, 256, 1040, 1100, 32, "bf16", False),   # rows wider than one 1024-column chunk
    (33, 3, 8, 40, 40, 32, "f32", True),            # small integers: exact ties and zero distances
    (31, 2, 16, 100, 37, 16, "bf16", True),
    (17, 1, 8, 5, 3, 3, "f32", False),              # k = |C'|
    (64, 1, 32, 512, 512, 8, "f32", True),          # 4 split blocks per half, ties across them
    (50, 2, 64, 600, 520, 16, "bf16", False),       # 2 split blocks per half
]


@pytest.mark.parametrize("T,h,dq,nk,nk2,k,dtype,integer", IDW_SCORE_CASES)
def test_idw_score_topk_stage(T, h, dq, nk, nk2, k, dtype, integer):
    note(f"idw score_topk T={T} h={h} dq={dq} nk={nk}/{nk2} k={k} {dtype} int={integer}")
    half = dq // 2
    if integer:
        q = pi.random_ints(12, 0, (T, h * dq), -1, 1, dtype=dtype)
        C = pi.random_ints(12, 1, (h, nk, half), -1, 1, dtype=dtype)
        Cp = pi.random_ints(12, 2, (h, nk2, half), -1, 1, dtype=dtype)
        # some query halves equal a sub-key: zero distances, scored at the floor
        for t in range(0, T, 3):
            hh = t % h
            q[t, hh * dq:hh * dq + half] = C[hh, t % nk]
            q[t, hh * dq + half:(hh + 1) * dq] = Cp[hh, (t + 1) % nk2]
    else:
        q = pi.random_array(12, 0, (T, h * dq), dtype=dtype, std=half ** -0.5)
        C = pi.random_array(12, 1, (h, nk, half), dtype=dtype, std=half ** -0.5)
        Cp = pi.random_array(12, 2, (h, nk2, half), dtype=dtype, std=half ** -0.5)
    cfg = _cfg(T=T, heads=h, dq=dq, n_keys=nk, n_keys2=nk2, topk=k, dtype=dtype, d_value=16)
    layer = layer_for(cfg, score="idw")
    from product_key_memory_pkm_amd import pkm_stage_score_topk
    si = torch.empty((T, h, 2, k), dtype=torch.int32, device="cuda")
    ss = torch.empty((T, h, 2, k), dtype=torch.float32, device="cuda")
    pkm_stage_score_topk(layer.handle, T, to_dev(q), to_dev(C), to_dev(Cp), si, ss, layer.workspace(T, False))
    torch.cuda.synchronize()
    si, ss = si.cpu().numpy(), ss.cpu().numpy()
    qd, Cd, Cpd = O.decode(q, dtype), O.decode(C, dtype), O.decode(Cp, dtype)
    q1, q2 = O.split_heads(qd, h, dq)
    s1, s2 = O.subkey_scores_idw(q1, q2, Cd, Cpd)
    zero_dist = 0
    for p, s, qh, K in ((0, s1, q1, Cd), (1, s2, q2, Cpd)):
        kk = min(k + 1, s.shape[-1])
        oi, ov = O.topk_sorted(s, kk)
        G = si[:, :, p, :]
        slack = None if integer else _half_slack(qh, K, ov[..., k - 1])
        valid, exact_set, exact_order = P.check_selection(
            G, oi, ov, lambda r: np.take_along_axis(s, r, axis=-1), s.shape[-1], k, slack)
        assert valid.all(), f"half {p}: {np.argwhere(~valid)[:5]}"
        ref = np.take_along_axis(s, G.astype(np.int64), axis=-1)
        if integer:
            assert exact_order.all()
            # -1/2 logf of an exact integer (or of the floor): logf's rounding only
            np.testing.assert_allclose(ss[:, :, p, :], ov[..., :k], rtol=4 * 2.0 ** -24, atol=1e-7)
            zero_dist += int((ov[..., :k] == -0.5 * np.log(O.IDW_FLOOR)).sum())
        else:
            assert exact_set.mean() > 0.99
            d2 = np.exp(-2.0 * ref)
            E = _u_bound(qh, K)[..., None]
            bound = E / np.maximum(d2 - E, 1e-30) + 4 * 2.0 ** -24 * np.abs(ref) + 1e-7
            assert (np.abs(ss[:, :, p, :] - ref) <= bound).all(), np.abs(ss[:, :, p, :] - ref).max()
    if integer:
        assert zero_dist > 0, "the integer case should hit the distance floor"


# ---------------------------------------------------------------------------
# pkm_forward with IDW scores (query projection, scoring, merge, gather)
# ---------------------------------------------------------------------------
def test_forward_with_idw_scores_end_to_end():
    from tests.test_gpu_forward import forward_check
    cfg = _cfg(T=300, d=64, heads=2, dq=64, n_keys=48, n_keys2=40, topk=16, d_value=32, dtype="f32", bn=True,
               seed=31)
    note(f"forward idw: {cfg}")
    inp = pi.make_inputs(cfg)
    layer = layer_for(cfg, score="idw")
    dev = upload(inp)
    y, saved = layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"])
    torch.cuda.synchronize()
    gpu = {"q": P.to_f64(saved["q"]), "idx": saved["idx"].cpu().numpy(), "w": saved["w"].cpu().numpy(),
           "y": P.to_f64(y)}
    stats = forward_check(cfg, inp, gpu, score="idw")
    assert stats["exact_set"] > 0.999


# ---------------------------------------------------------------------------
# FwPKM memorization chunk
# ---------------------------------------------------------------------------
def _chunk_inputs(cfg, integer_keys: bool, tag: int = 0):
    half = cfg.dq // 2
    s = cfg.seed
    if integer_keys:
        q = pi.random_ints(s, 10 + tag, (cfg.T, cfg.F), -1, 1, dtype=cfg.dtype)
        C = pi.random_ints(s, 11, (cfg.heads, cfg.n_keys, half), -1, 1, dtype=cfg.dtype)
        Cp = pi.random_ints(s, 12, (cfg.heads, cfg.n_keys2, half), -1, 1, dtype=cfg.dtype)
    else:
        q = pi.random_array(s, 10 + tag, (cfg.T, cfg.F), dtype=cfg.dtype, std=half ** -0.5)
        C = pi.random_array(s, 11, (cfg.heads, cfg.n_keys, half), dtype=cfg.dtype, std=half ** -0.5)
        Cp = pi.random_array(s, 12, (cfg.heads, cfg.n_keys2, half), dtype=cfg.dtype, std=half ** -0.5)
    target = pi.random_array(s, 14 + tag, (cfg.T, cfg.d_value), dtype=cfg.dtype)
    return q, C, Cp, target


def _values(cfg):
    return pi.random_array(cfg.seed, 13, (cfg.slots, cfg.d_value), dtype=cfg.dtype, std=cfg.d_value ** -0.5)


def _run_chunk(layer, q, C, Cp, V_dev, target, lr):
    y, idx, w = layer.fwpkm_chunk(to_dev(q), to_dev(C), to_dev(Cp), V_dev, to_dev(target), lr)
    torch.cuda.synchronize()
    return P.to_f64(y), idx.cpu().numpy(), w.cpu().numpy()


def _check_chunk(cfg, q, C, Cp, V_in, target, lr, y_g, G, w_g, V_g, integer, prior_bad=None, V_prev_g=None):
    """Compare one GPU chunk with O.fwpkm_chunk on the same V_in.

    Integer keys give exact ties between full keys (a full key scores -1/2 log(d1^2 d2^2), and
    different products of squared distances can be equal): any of the tied keys is a correct pick,
    so the selected sets may differ there.  Tokens whose sets differ on some head are compared on
    what is unique (valid selection, weights and y of their own selection); the rows they write,
    and ``prior_bad`` (rows an earlier chunk left different), are left out of the value comparison,
    and tokens reading ``prior_bad`` rows out of the comparison of y.  Rows no lookup selects must
    keep the GPU's previous values bit for bit (``V_prev_g``, default V_in).
    Returns (the oracle's V after the write, float64; rows left out of the comparison)."""
    y_o, V_o, sel = O.fwpkm_chunk(cfg, q, C, Cp, V_in, target, lr)
    qd, Cd, Cpd = O.decode(q, cfg.dtype), O.decode(C, cfg.dtype), O.decode(Cp, cfg.dtype)
    q1, q2 = O.split_heads(qd, cfg.heads, cfg.dq)
    s1, s2 = O.subkey_scores_idw(q1, q2, Cd, Cpd)

    def score_of(r):
        return P.full_scores(r.astype(np.int64), s1, s2, cfg.n_keys2)

    slack = None
    if not integer:
        # a full key near the k-th best pairs sub-keys from the halves' top-k lists, the closest of which
        # (the first entry) has the largest score error; each side of a swap carries one such error
        slack = 2 * (_score_err(q1, Cd, sel["sub_val1"]) + _score_err(q2, Cpd, sel["sub_val2"]))
    valid, exact_set, exact_order = P.check_selection(G, sel["rows_k1"], sel["scores_k1"], score_of, cfg.slots,
                                                      cfg.topk, slack)
    assert valid.all(), f"invalid selections at {np.argwhere(~valid)[:5].tolist()}"
    tol = P.TOL[cfg.dtype]
    w_ref = O.softmax(score_of(G), cfg.temperature)
    assert np.abs(w_g - w_ref).max() <= tol * max(1e-3, float(np.abs(w_ref).max()))
    prior_bad = np.zeros(0, np.int64) if prior_bad is None else prior_bad
    reads_bad = np.isin(G.reshape(G.shape[0], -1), prior_bad).any(-1)
    # y of the GPU's own selection, read before the write
    y_own = O.round_to_storage(O.gather_sum(G.astype(np.int64), w_ref, V_in, cfg.dtype), cfg.dtype)
    ok = ~reads_bad
    assert P.row_rel_err(y_g[ok], y_own[ok]).max() <= tol
    same = exact_set.all(-1)                          # tokens whose selected sets agree on every head
    assert same.mean() > (0.5 if integer else 0.98)
    cmp = same & ok
    assert cmp.any()
    assert P.row_rel_err(y_g[cmp], y_o[cmp]).max() <= tol
    # rows written by a token whose set differs, or by one that read a differing row, are left out
    bad_tok = ~cmp
    bad_rows = np.union1d(G[bad_tok].reshape(-1), sel["rows"][bad_tok].reshape(-1)).astype(np.int64)
    bad_rows = np.union1d(bad_rows, prior_bad)
    touched = np.union1d(G.reshape(-1), sel["rows"].reshape(-1)).astype(np.int64)
    Vin = O.decode(V_in, cfg.dtype)
    untouched = np.ones(cfg.slots, bool)
    untouched[touched] = False
    V_prev = Vin if V_prev_g is None else V_prev_g
    np.testing.assert_array_equal(V_g[untouched], V_prev[untouched])   # no other row is written
    good = np.setdiff1d(touched, bad_rows)
    assert good.size > 0.5 * touched.size
    # the write is V - lr * g: compare it against the size of the row and of the step
    step = np.abs(V_o[good] - Vin[good]).max(axis=1)
    den = np.maximum(np.abs(V_o[good]).max(axis=1), 1e-30)
    err = np.abs(V_g[good] - V_o[good]).max(axis=1) / den
    assert err.max() <= tol, err.max()
    assert (step > 0).mean() > 0.9 if lr > 0 else (step == 0).all()
    return V_o, bad_rows


FWPKM_CASES = {
    "small_f32": (_cfg(T=200, heads=2, dq=32, n_keys=24, n_keys2=20, topk=8, d_value=48, seed=41), False, 0.5),
    "ragged_bf16": (_cfg(T=77, heads=3, dq=48, n_keys=50, n_keys2=33, topk=16, d_value=40, dtype="bf16",
                         seed=42), False, 0.25),
    # integer keys: exact full-key ties; a sparse table keeps most written rows comparable
    "int_keys": (_cfg(T=64, heads=1, dq=16, n_keys=32, n_keys2=32, topk=4, d_value=32, seed=43), True, 1.0),
    # every row gets hundreds of lookups: the per-row sums run in chunks and a combine pass
    "hot": (_cfg(T=2048, heads=2, dq=32, n_keys=8, n_keys2=8, topk=8, d_value=40, seed=44), False, 0.01),
    # 8000 lookups (one-workgroup grouping) over 16 rows: every row's sum runs in chunks
    "hot_small": (_cfg(T=2000, heads=1, dq=16, n_keys=4, n_keys2=4, topk=4, d_value=32, seed=49), False, 0.01),
    "one_token": (_cfg(T=1, heads=1, dq=16, n_keys=8, n_keys2=8, topk=4, d_value=16, dtype="bf16", seed=45),
                  False, 1.0),
    "lr_zero": (_cfg(T=50, heads=1, dq=32, n_keys=16, n_keys2=16, topk=8, d_value=32, seed=46), False, 0.0),
    # a 512-token chunk over 1024 x 1024 slots with k = 8 (the fast-weight page's chunking and sparsity)
    "wide": (_cfg(T=512, heads=1, dq=128, n_keys=1024, n_keys2=1024, topk=8, d_value=16, seed=47), False, 0.5),
}


@pytest.mark.parametrize("name", list(FWPKM_CASES))
def test_fwpkm_chunk(name):
    cfg, integer, lr = FWPKM_CASES[name]
    note(f"fwpkm chunk {name}: {cfg} lr={lr}")
    q, C, Cp, target = _chunk_inputs(cfg, integer)
    V = _values(cfg)
    layer = layer_for(cfg, score="idw")
    V_dev = to_dev(V)
    y_g, G, w_g = _run_chunk(layer, q, C, Cp, V_dev, target, lr)
    _check_chunk(cfg, q, C, Cp, V, target, lr, y_g, G, w_g, P.to_f64(V_dev), integer)


@pytest.mark.parametrize("integer", [False, True])
def test_fwpkm_chunks_in_sequence(integer):
    # the second chunk reads what the first one wrote: compare against the oracle's own sequence
    cfg = _cfg(T=64, heads=1, dq=16, n_keys=32, n_keys2=32, topk=8, d_value=24, seed=48)
    note(f"fwpkm two chunks (integer keys {integer}): {cfg}")
    q1, C, Cp, t1 = _chunk_inputs(cfg, integer, tag=0)
    q2, _, _, t2 = _chunk_inputs(cfg, integer, tag=5)
    V = _values(cfg)
    layer = layer_for(cfg, score="idw")
    V_dev = to_dev(V)
    y1, G1, w1 = _run_chunk(layer, q1, C, Cp, V_dev, t1, 0.5)
    V1_o, bad1 = _check_chunk(cfg, q1, C, Cp, V, t1, 0.5, y1, G1, w1, P.to_f64(V_dev), integer)
    V1 = V1_o.astype(np.float32)                      # the oracle's fp32 table after the first write
    V1_g = P.to_f64(V_dev)
    y2, G2, w2 = _run_chunk(layer, q2, C, Cp, V_dev, t2, 0.5)
    _check_chunk(cfg, q2, C, Cp, V1, t2, 0.5, y2, G2, w2, P.to_f64(V_dev), integer, prior_bad=bad1,
                 V_prev_g=V1_g)
    # and the second chunk depends on the write before it
    y2_fresh, _, _ = O.fwpkm_chunk(cfg, q2, C, Cp, V, t2, 0.5)
    y2_seq, _, _ = O.fwpkm_chunk(cfg, q2, C, Cp, V1, t2, 0.5)
    assert P.row_rel_err(y2_fresh, y2_seq).max() > 1e-3


def test_fwpkm_chunk_is_deterministic():
    cfg, integer, lr = FWPKM_CASES["hot"]
    note("fwpkm chunk determinism")
    q, C, Cp, target = _chunk_inputs(cfg, integer)
    V = _values(cfg)
    layer = layer_for(cfg, score="idw")
    outs = []
    for _ in range(2):
        V_dev = to_dev(V)
        y, G, w = _run_chunk(layer, q, C, Cp, V_dev, target, lr)
        outs.append((y, G, w, P.to_f64(V_dev)))
    for a, b in zip(*outs):
        np.testing.assert_array_equal(a, b)


def test_fwpkm_chunk_at_the_benchmark_configuration():
    # the launch configuration bench.py times: 512 tokens, one head, dq = 512, 1024 x 1024 slots,
    # k = 8, 1600-wide bf16 value rows; the oracle reads only the selected rows (dense=False)
    cfg = _cfg(T=512, heads=1, dq=512, n_keys=1024, n_keys2=1024, topk=8, d_value=1600, dtype="bf16", seed=50)
    lr = 0.1
    note(f"fwpkm chunk at the benchmark configuration: {cfg}")
    half = cfg.dq // 2
    q, target = pi.fwpkm_stream(cfg.seed, cfg.T, cfg.dq, cfg.d_value, cfg.dtype)
    C = pi.random_array(cfg.seed, 11, (1, cfg.n_keys, half), dtype=cfg.dtype, std=half ** -0.5)
    Cp = pi.random_array(cfg.seed, 12, (1, cfg.n_keys2, half), dtype=cfg.dtype, std=half ** -0.5)
    V = _values(cfg)
    layer = layer_for(cfg, score="idw")
    V_dev = to_dev(V)
    y_g, G, w_g = _run_chunk(layer, q, C, Cp, V_dev, target, lr)
    y_o, (ids, rows_new), sel = O.fwpkm_chunk(cfg, q, C, Cp, V, target, lr, dense=False)
    qd, Cd, Cpd = O.decode(q, cfg.dtype), O.decode(C, cfg.dtype), O.decode(Cp, cfg.dtype)
    q1, q2 = O.split_heads(qd, 1, cfg.dq)
    s1, s2 = O.subkey_scores_idw(q1, q2, Cd, Cpd)

    def score_of(r):
        return P.full_scores(r.astype(np.int64), s1, s2, cfg.n_keys2)

    slack = 2 * (_score_err(q1, Cd, sel["sub_val1"]) + _score_err(q2, Cpd, sel["sub_val2"]))
    valid, exact_set, _ = P.check_selection(G, sel["rows_k1"], sel["scores_k1"], score_of, cfg.slots, cfg.topk,
                                            slack)
    assert valid.all()
    tol = P.TOL[cfg.dtype]
    w_ref = O.softmax(score_of(G), cfg.temperature)
    assert np.abs(w_g - w_ref).max() <= tol * max(1e-3, float(np.abs(w_ref).max()))
    same = exact_set.all(-1)
    assert same.mean() > 0.98
    assert P.row_rel_err(y_g[same], y_o[same]).max() <= tol
    # value rows: the written rows (those of tokens whose sets agree), and untouched rows unchanged
    bad = np.union1d(G[~same].reshape(-1), sel["rows"][~same].reshape(-1))
    good = ~np.isin(ids, bad)
    assert good.mean() > 0.98
    V_after = V_dev[torch.from_numpy(ids[good]).cuda()]
    err = P.row_rel_err(P.to_f64(V_after), rows_new[good])
    assert err.max() <= tol, err.max()
    assert (rows_new[good] != O.decode(V[ids[good]], cfg.dtype)).any(axis=1).mean() > 0.9
    g = np.random.default_rng(0)
    sample = np.setdiff1d(g.integers(0, cfg.slots, 200_000), np.union1d(ids, G.reshape(-1)))
    np.testing.assert_array_equal(V_dev[torch.from_numpy(sample).cuda()].cpu().view(torch.int16).numpy(),
                                  V[sample].view(np.int16))


BATCH_CASES = [
    # streams, tokens per stream, heads, dq, nk, k, d_value, dtype
    (3, 40, 2, 16, 12, 4, 24, "f32"),            # 960 lookups: one-workgroup grouping
    (4, 512, 1, 32, 64, 8, 32, "bf16"),          # 16384 lookups: a workgroup per stream, 4 x 4096 slots
    (3, 2000, 1, 16, 4, 4, 32, "f32"),           # a workgroup per stream, ~500 lookups per row: long runs
    (64, 64, 2, 16, 16, 8, 16, "f32"),           # 64 streams of 1024 lookups
    (2, 4608, 1, 16, 64, 2, 16, "f32"),          # 9216 lookups per stream: above one workgroup, radix sort
]


@pytest.mark.parametrize("streams,tps,h,dq,nk,k,dv,dtype", BATCH_CASES)
def test_fwpkm_chunk_batch_of_streams(streams, tps, h, dq, nk, k, dv, dtype):
    # each stream is its own chunk on its own table: compare stream by stream with the oracle
    cfg = _cfg(T=tps, heads=h, dq=dq, n_keys=nk, n_keys2=nk, topk=k, d_value=dv, dtype=dtype, seed=51)
    lr = 0.5
    note(f"fwpkm chunk, {streams} streams of {tps} tokens: {cfg}")
    half = dq // 2
    C = pi.random_array(cfg.seed, 11, (h, nk, half), dtype=dtype, std=half ** -0.5)
    Cp = pi.random_array(cfg.seed, 12, (h, nk, half), dtype=dtype, std=half ** -0.5)
    qs, ts, Vs = [], [], []
    for b in range(streams):
        qs.append(pi.random_array(cfg.seed, 20 + b, (tps, h * dq), dtype=dtype, std=half ** -0.5))
        ts.append(pi.random_array(cfg.seed, 40 + b, (tps, dv), dtype=dtype))
        Vs.append(pi.random_array(cfg.seed, 60 + b, (cfg.slots, dv), dtype=dtype, std=dv ** -0.5))
    layer = layer_for(cfg, score="idw")
    V_dev = to_dev(np.concatenate(Vs))
    y, idx, w = layer.fwpkm_chunk(to_dev(np.concatenate(qs)), to_dev(C), to_dev(Cp), V_dev,
                                  to_dev(np.concatenate(ts)), lr, streams=streams)
    torch.cuda.synchronize()
    y, idx, w, V_all = P.to_f64(y), idx.cpu().numpy(), w.cpu().numpy(), P.to_f64(V_dev)
    for b in range(streams):
        tok = slice(b * tps, (b + 1) * tps)
        rows = slice(b * cfg.slots, (b + 1) * cfg.slots)
        G = idx[tok]
        assert ((G >= b * cfg.slots) & (G < (b + 1) * cfg.slots)).all(), "a stream addressed another's table"
        _check_chunk(cfg, qs[b], C, Cp, Vs[b], ts[b], lr, y[tok], G - b * cfg.slots, w[tok], V_all[rows], False)


CALLS_CASES = [
    # streams, tokens per stream and call, calls, heads, dq, nk, k, d_value, dtype
    (1, 64, 4, 1, 16, 32, 8, 24, "f32"),         # one stream: every call's grouping up front
    (1, 512, 3, 1, 64, 64, 8, 32, "bf16"),       # the benchmark's chunk length
    (1, 2000, 3, 1, 16, 4, 4, 32, "f32"),        # 16 slots: runs of ~500 lookups (each call's long-run plan)
    (1, 4608, 2, 1, 16, 64, 2, 16, "f32"),       # 9216 lookups per call: grouped call by call (radix sort)
    (3, 40, 3, 2, 16, 12, 4, 24, "f32"),         # a batch of streams: the tables' offsets restart every call
    (2, 1000, 3, 1, 16, 4, 4, 32, "f32"),        # a batch whose calls have runs of ~250 lookups per row
    (2, 4608, 2, 1, 16, 64, 2, 16, "f32"),       # 9216 lookups per stream and call: the radix sort
]


@pytest.mark.parametrize("streams,tps,calls,h,dq,nk,k,dv,dtype", CALLS_CASES)
def test_fwpkm_chunks_equal_the_calls_in_sequence(streams, tps, calls, h, dq, nk, k, dv, dtype):
    # pkm_fwpkm_chunks selects all tokens first, then writes slice by slice: every output and the final
    # table must be those of pkm_fwpkm_chunk called on the slices one after another, bit for bit
    cfg = _cfg(T=tps, heads=h, dq=dq, n_keys=nk, n_keys2=nk, topk=k, d_value=dv, dtype=dtype, seed=53)
    lr = 0.5
    call_T = streams * tps
    T = calls * call_T
    note(f"fwpkm chunks: {calls} calls of {streams} x {tps} tokens: {cfg}")
    half = dq // 2
    C = to_dev(pi.random_array(cfg.seed, 11, (h, nk, half), dtype=dtype, std=half ** -0.5))
    Cp = to_dev(pi.random_array(cfg.seed, 12, (h, nk, half), dtype=dtype, std=half ** -0.5))
    q = to_dev(pi.random_array(cfg.seed, 20, (T, h * dq), dtype=dtype, std=half ** -0.5))
    target = to_dev(pi.random_array(cfg.seed, 40, (T, dv), dtype=dtype))
    V0 = to_dev(pi.random_array(cfg.seed, 60, (streams * cfg.slots, dv), dtype=dtype, std=dv ** -0.5))
    layer = layer_for(cfg, score="idw")
    V_seq = V0.clone()
    seq = [layer.fwpkm_chunk(q[j * call_T:(j + 1) * call_T], C, Cp, V_seq, target[j * call_T:(j + 1) * call_T],
                             lr, streams=streams) for j in range(calls)]
    seq = [tuple(t.clone() for t in r) for r in seq]
    V_one = V0.clone()
    y, idx, w = layer.fwpkm_chunks(q, C, Cp, V_one, target, lr, call_T, streams=streams)
    torch.cuda.synchronize()
    assert torch.equal(idx, torch.cat([r[1] for r in seq])), "selections differ"
    assert torch.equal(w, torch.cat([r[2] for r in seq])), "weights differ"
    assert torch.equal(y, torch.cat([r[0] for r in seq])), "outputs differ"
    assert torch.equal(V_one, V_seq), "tables differ"
    assert not torch.equal(V_one, V0)
