"""The chunked, threaded helpers of tests/parity.py against the oracle's own whole-batch functions (CPU).

The full-size GPU tests run the oracle's per-token steps over token chunks in threads; these checks show
that the chunking changes nothing but the order of floating-point sums."""
import numpy as np

import pkm_inputs as pi
from oracle import pkm_oracle as O
from tests import parity as P


def _case(dtype, bn, tau=1.0):
    cfg = pi.custom(T=300, d=24, heads=3, dq=16, n_keys=20, n_keys2=13, topk=6, d_value=12, dtype=dtype, bn=bn,
                    seed=61, temperature=tau)
    return cfg, pi.make_inputs(cfg, with_dy=True)


def test_lookup_chunks_equals_lookup():
    cfg, inp = _case("bf16", True)
    ref = O.forward(cfg, inp, keep_tables=True)
    C, Cp = O.decode(inp["C"], cfg.dtype), O.decode(inp["Cp"], cfg.dtype)
    sel = P.lookup_chunks(cfg, ref["q"], C, Cp, chunk=37)
    for key in ("rows", "scores", "w", "rows_k1", "scores_k1", "s1", "s2", "sub_idx1", "sub_idx2"):
        np.testing.assert_array_equal(sel[key], ref[key], err_msg=key)


def test_scores_at_equals_table_lookup():
    cfg, inp = _case("f32", True)
    ref = O.forward(cfg, inp, keep_tables=True)
    C, Cp = O.decode(inp["C"], cfg.dtype), O.decode(inp["Cp"], cfg.dtype)
    G = ref["rows_k1"]
    got = P.scores_at(cfg, ref["q"], C, Cp, G, chunk=41)
    np.testing.assert_array_equal(got, P.full_scores(G, ref["s1"], ref["s2"], cfg.n_keys2))
    np.testing.assert_allclose(got, ref["scores_k1"], rtol=1e-13, atol=1e-13)


def test_backward_chunks_equals_backward():
    for dtype, bn, tau in (("f32", True, 1.0), ("bf16", True, 0.5), ("f32", False, 2.0)):
        cfg, inp = _case(dtype, bn, tau)
        fwd = O.forward(cfg, inp)
        want = O.backward(cfg, inp, fwd, inp["dY"])
        got = P.backward_chunks(cfg, inp, fwd, inp["dY"], chunk=64)
        for key in ("dw", "ds", "dq", "dq_pre", "dC", "dCp", "dWq", "dx", "dgamma", "dbeta"):
            if want[key] is None:
                assert got[key] is None
                continue
            np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-12 * np.abs(want[key]).max(),
                                       err_msg=key)


def test_backward_chunks_on_a_token_subset():
    # tokens outside the subset have a zero upstream gradient: the subset run equals the full one
    cfg, inp = _case("bf16", True, 0.7)
    fwd = O.forward(cfg, inp)
    tok = np.arange(3, cfg.T, 7)
    dY = inp["dY"].copy()
    keep = np.zeros(cfg.T, bool)
    keep[tok] = True
    dY[~keep] = 0
    want = O.backward(cfg, inp, fwd, dY)
    got = P.backward_chunks(cfg, inp, fwd, dY, chunk=16, tokens=tok)
    for key in ("dw", "ds", "dq", "dq_pre", "dC", "dCp", "dWq", "dx", "dgamma", "dbeta"):
        np.testing.assert_allclose(got[key], want[key], rtol=1e-12, atol=1e-12 * np.abs(want[key]).max(),
                                   err_msg=key)
    sub = dict(fwd, rows=fwd["rows"][tok], w=fwd["w"][tok], q=fwd["q"][tok])
    got2 = P.backward_chunks(cfg, inp, sub, dY, chunk=16, tokens=tok)
    np.testing.assert_allclose(got2["dWq"], want["dWq"], rtol=1e-12, atol=1e-12 * np.abs(want["dWq"]).max())
