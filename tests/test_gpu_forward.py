"""GPU parity of the forward steps (a1-a6) against the fp64 CPU oracle.

Every test feeds both sides the same seeded inputs (``pkm_inputs``) and calls
the HIP path through the C ABI binding.  Rules and tolerances: tests/parity.py.
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
    base = dict(T=64, d=64, heads=1, dq=32, n_keys=32, n_keys2=32, topk=8, d_value=64, dtype="f32", bn=False,
                seed=3)
    base.update(kw)
    return pi.custom(**base)


# ---------------------------------------------------------------------------
# a6: gather-sum on seeded selections
# ---------------------------------------------------------------------------
GATHER_CASES = [
    # T, heads, k, rows, d_value, dtype
    (37, 3, 5, 100, 24, "f32"),
    (64, 4, 32, 5000, 1600, "bf16"),
    (129, 2, 7, 300, 8, "bf16"),       # one 16-byte vector per row
    (33, 1, 3, 50, 2048, "bf16"),      # 256 vectors per row: 4 per lane
    (70, 4, 32, 4096, 512, "f32"),
    (5, 8, 32, 777, 1024, "bf16"),     # 256 rows per token
    (3, 1, 1, 10, 64, "f32"),          # k = 1
]


@pytest.mark.parametrize("T,h,k,nrows,dv,dtype", GATHER_CASES)
def test_gather_stage(T, h, k, nrows, dv, dtype):
    note(f"gather T={T} h={h} k={k} rows={nrows} dv={dv} {dtype}")
    rows, w = pi.random_selection(T + nrows, T, h, k, nrows)
    V = pi.random_array(7, 1, (nrows, dv), dtype=dtype)
    # a layer whose slot count covers nrows; only (h, k, d_value, dtype) matter for the gather
    nk = int(np.ceil(np.sqrt(nrows)))
    cfg = _cfg(heads=h, topk=k, n_keys=max(nk, k), n_keys2=max(nk, k), d_value=dv, dtype=dtype,
               d=16 if dtype == "bf16" else 8, dq=32)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_gather
    y = torch.empty((T, dv), dtype=layer.storage, device="cuda")
    # the table holds the layer's |C|*|C'| rows (the lookups use the first nrows)
    Vt = np.concatenate([V, np.zeros((cfg.slots - nrows, dv), dtype=V.dtype)])
    pkm_stage_gather(layer.handle, T, to_dev(rows), to_dev(w), to_dev(Vt), y)
    torch.cuda.synchronize()
    ref = O.gather_sum(rows, w.astype(np.float64), V, dtype)
    err = P.row_rel_err(P.to_f64(y), ref)
    # fp32 accumulation of h*k terms; bf16 output rounding dominates for bf16
    tol = 1e-5 if dtype == "f32" else 8e-3
    assert err.max() <= tol, err.max()
    if k == 1 and h == 1 and dtype == "f32":
        # one row with weight 1: an exact copy
        np.testing.assert_array_equal(P.to_f64(y), V[rows[:, 0, 0]].astype(np.float64))


# ---------------------------------------------------------------------------
# a3 + a4: scores and per-half top-k on a seeded query
# ---------------------------------------------------------------------------
SCORE_CASES = [
    # T, heads, dq, nk, nk2, k, dtype, integer
    (100, 2, 32, 32, 48, 8, "f32", False),
    (257, 4, 256, 256, 256, 32, "f32", False),
    (75, 4, 512, 1024, 1024, 32, "bf16", False),
    (40, 2, 512, 2048, 2000, 32, "bf16", False),
    (50, 1, 16, 8, 64, 8, "bf16", False),
    (33, 3, 32, 40, 40, 32, "f32", True),      # small integers: many exact ties
    (31, 2, 64, 100, 37, 32, "bf16", True),
    (17, 1, 8, 5, 3, 3, "f32", False),         # k = |C'|
    # rows wider than one chunk of 1024 columns: the chunk top-k lists are merged
    (60, 2, 256, 1040, 1100, 32, "bf16", False),  # last chunk narrower than k
    (30, 2, 32, 1300, 40, 32, "f32", True),       # ties across chunks: lowest index wins
    (20, 1, 512, 1024, 1024, 16, "f32", False),   # fp32 with wide halves: 512-column chunks
    # launches too small for the chip split each half's sub-keys over 2 or 4 blocks and merge their lists
    (40, 1, 32, 256, 512, 8, "f32", False),       # 4 splits
    (33, 3, 32, 300, 280, 8, "f32", True),        # 4 splits, ties across splits: lowest index wins
    (20, 2, 64, 512, 512, 16, "bf16", False),     # 2 splits
    (25, 1, 16, 130, 129, 4, "bf16", True),       # splits of unequal width
    # bf16 codebooks with many tiles, ragged codebooks, wide halves and heavy ties
    (4096, 4, 512, 1024, 1024, 32, "bf16", False),  # the paper's key shape, many tiles
    (1500, 2, 256, 700, 600, 16, "bf16", False),    # ragged codebooks, unequal halves
    (300, 1, 64, 400, 300, 8, "bf16", False),       # k = 8, one head
    (257, 2, 1024, 2048, 1500, 32, "bf16", False),  # half of 512 dims, 2048 sub-keys, ragged token tail
    (2000, 2, 512, 1024, 1024, 32, "bf16", True),   # heavy ties across the whole codebook
    (100, 2, 512, 2048, 2048, 32, "bf16", True),    # the same with 2048 sub-keys and few tokens
]


def _score_tables(q, C, Cp, heads, dq):
    q1, q2 = O.split_heads(q, heads, dq)
    return O.subkey_scores(q1, q2, C, Cp)


@pytest.mark.parametrize("T,h,dq,nk,nk2,k,dtype,integer", SCORE_CASES)
def test_score_topk_stage(T, h, dq, nk, nk2, k, dtype, integer):
    note(f"score_topk T={T} h={h} dq={dq} nk={nk}/{nk2} k={k} {dtype} int={integer}")
    half = dq // 2
    if integer:
        q = pi.random_ints(11, 0, (T, h * dq), -2, 2, dtype=dtype)
        C = pi.random_ints(11, 1, (h, nk, half), -1, 1, dtype=dtype)
        Cp = pi.random_ints(11, 2, (h, nk2, half), -1, 1, dtype=dtype)
    else:
        q = pi.random_array(11, 0, (T, h * dq), dtype=dtype)
        C = pi.random_array(11, 1, (h, nk, half), dtype=dtype, std=half ** -0.5)
        Cp = pi.random_array(11, 2, (h, nk2, half), dtype=dtype, std=half ** -0.5)
    cfg = _cfg(T=T, heads=h, dq=dq, n_keys=nk, n_keys2=nk2, topk=k, dtype=dtype, d=16, d_value=16)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_score_topk
    si = torch.empty((T, h, 2, k), dtype=torch.int32, device="cuda")
    ss = torch.empty((T, h, 2, k), dtype=torch.float32, device="cuda")
    pkm_stage_score_topk(layer.handle, T, to_dev(q), to_dev(C), to_dev(Cp), si, ss, layer.workspace(T, False))
    torch.cuda.synchronize()
    si, ss = si.cpu().numpy(), ss.cpu().numpy()
    qd, Cd, Cpd = O.decode(q, dtype), O.decode(C, dtype), O.decode(Cp, dtype)
    s1, s2 = _score_tables(qd, Cd, Cpd, h, dq)
    for p, s in ((0, s1), (1, s2)):
        kk = min(k + 1, s.shape[-1])
        oi, ov = O.topk_sorted(s, kk)
        G = si[:, :, p, :]
        valid, exact_set, exact_order = P.check_selection(
            G, oi, ov, lambda r: np.take_along_axis(s, r, axis=-1), s.shape[-1], k)
        assert valid.all(), f"half {p}: {np.argwhere(~valid)[:5]}"
        if integer:
            # integer inputs: every sum is exact in fp32, so the lowest-index rule decides ties exactly
            assert exact_order.all()
            np.testing.assert_array_equal(ss[:, :, p, :], ov[..., :k].astype(np.float32))
        else:
            assert exact_set.mean() > 0.99
            # returned scores are the GPU's fp32 sums of the selected sub-keys
            ref = np.take_along_axis(s, G.astype(np.int64), axis=-1)
            np.testing.assert_allclose(ss[:, :, p, :], ref, rtol=2e-5, atol=2e-5 * np.abs(ref).max())


# ---------------------------------------------------------------------------
# a5: candidate merge, top-k, softmax on seeded sorted lists
# ---------------------------------------------------------------------------
MERGE_CASES = [
    # T, heads, k, nk, nk2, integer, tau
    (200, 4, 32, 1024, 1024, False, 1.0),
    (97, 2, 8, 32, 48, False, 0.5),
    (64, 3, 32, 64, 40, True, 1.0),
    (50, 1, 1, 5, 7, False, 1.0),
    (33, 2, 17, 300, 20, True, 2.0),
]


@pytest.mark.parametrize("T,h,k,nk,nk2,integer,tau", MERGE_CASES)
def test_merge_softmax_stage(T, h, k, nk, nk2, integer, tau):
    note(f"merge T={T} h={h} k={k} nk={nk}/{nk2} int={integer} tau={tau}")
    si, ss = pi.random_sublists(5, T, h, k, nk, nk2, integer=integer)
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=nk, n_keys2=nk2, temperature=tau, d=8, d_value=8, dq=8)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_merge_softmax
    idx = torch.empty((T, h, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    sc = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    pkm_stage_merge_softmax(layer.handle, T, to_dev(si), to_dev(ss), idx, w, sc)
    torch.cuda.synchronize()
    idx, w, sc = idx.cpu().numpy(), w.cpu().numpy(), sc.cpu().numpy()
    v1 = ss[:, :, 0, :].astype(np.float64)
    v2 = ss[:, :, 1, :].astype(np.float64)
    cs, cr = O.candidates(si[:, :, 0, :], v1, si[:, :, 1, :], v2, nk2)
    kk = min(k + 1, k * k)
    orows, oscores = O.select_topk(cs, cr, kk)
    lut = {}

    def score_of(r):
        # full-key score of a candidate row from the two lists (rows outside the k x k grid never occur)
        out = np.empty(r.shape)
        for t in range(T):
            for hh in range(h):
                m = dict(zip(cr[t, hh].tolist(), cs[t, hh].tolist()))
                out[t, hh] = [m.get(int(x), -np.inf) for x in r[t, hh]]
        return out

    valid, exact_set, exact_order = P.check_selection(idx, orows, oscores, score_of, nk * nk2, k)
    assert valid.all()
    if integer:
        assert exact_order.all()
    else:
        assert exact_set.all()
    ow = O.softmax(oscores[..., :k], tau)
    # weights compared where the selection is the oracle's, in the oracle's order
    sel = exact_order
    np.testing.assert_allclose(w[sel], ow[sel], rtol=2e-6, atol=1e-7)
    np.testing.assert_allclose(w.sum(-1), 1.0, atol=2e-6)
    assert (np.diff(w, axis=-1) <= 1e-7).all()


# ---------------------------------------------------------------------------
# a1 + a2: projection and BatchNorm
# ---------------------------------------------------------------------------
QUERY_CASES = [
    # T, d, heads, dq, dtype, bn
    (64, 64, 1, 32, "f32", False),
    (300, 128, 2, 32, "f32", True),
    (1000, 1600, 4, 512, "bf16", True),
    (77, 24, 3, 16, "bf16", True),
    (1, 16, 1, 16, "bf16", False),
]


@pytest.mark.parametrize("T,d,h,dq,dtype,bn", QUERY_CASES)
def test_query_stage(T, d, h, dq, dtype, bn):
    note(f"query T={T} d={d} h={h} dq={dq} {dtype} bn={bn}")
    cfg = _cfg(T=T, d=d, heads=h, dq=dq, dtype=dtype, bn=bn, n_keys=8, n_keys2=8, d_value=16, topk=4, seed=T)
    inp = pi.make_inputs(cfg)
    gamma = np.linspace(0.5, 1.5, cfg.F).astype(np.float32)
    beta = np.linspace(-0.3, 0.2, cfg.F).astype(np.float32)
    inp["gamma"], inp["beta"] = gamma, beta
    layer = layer_for(cfg)
    dev = upload(inp)
    saved = layer.alloc_saved(T)
    from product_key_memory_pkm_amd import pkm_stage_query
    pkm_stage_query(layer.handle, T, dev["x"], dev["Wq"], dev["gamma"], dev["beta"], saved, layer.workspace(T, False))
    torch.cuda.synchronize()
    ref = O.query(cfg, inp)
    qpre = P.to_f64(saved["q_pre"])
    assert P.fro_rel_err(qpre, ref["q_pre"]) <= 1e-6
    assert P.row_rel_err(qpre, ref["q_pre"]).max() <= (1e-5 if dtype == "f32" else 1e-5)
    q = P.to_f64(saved["q"])
    if bn:
        np.testing.assert_allclose(P.to_f64(saved["bn_mean"]), ref["mean"], rtol=1e-5,
                                   atol=1e-6 * np.abs(ref["q_pre"]).max())
        np.testing.assert_allclose(P.to_f64(saved["bn_rstd"]), 1 / np.sqrt(ref["var"] + cfg.bn_eps), rtol=2e-5)
    if dtype == "bf16":
        # q is the nearest bf16 of a value the two sides compute in different precision: equal or one ulp apart
        assert (np.abs(q - ref["q"]) <= P.q_allowed(q, ref["q"])).all()
        assert (q != ref["q"]).mean() < 0.01
    else:
        assert P.row_rel_err(q, ref["q"]).max() <= 1e-5


# ---------------------------------------------------------------------------
# whole forward
# ---------------------------------------------------------------------------
def forward_check(cfg, inp, gpu: dict, tokens=None, score="dot"):
    """Compare a GPU forward (q, idx, w, y as numpy) with the oracle on ``tokens`` (default all).

    The query is compared with the oracle's (bf16: equal or one ulp apart).  The selection is judged
    against the oracle's exact search with no slack: on the oracle's own query for fp32 storage, on the
    GPU's saved bf16 query for bf16 storage (the values the scores are computed from; the ulp choice is
    checked just above).  ``score`` "idw": fp32 storage only.  Returns the exact-set and exact-order
    shares, the oracle's forward and the search the selection was judged on."""
    assert score == "dot" or cfg.dtype == "f32"
    tok = np.arange(cfg.T) if tokens is None else np.asarray(tokens)
    ref = O.forward(cfg, inp, tokens=tok, keep_tables=cfg.dtype != "bf16", score=score)
    tol = P.TOL[cfg.dtype]
    q_g = gpu["q"][tok] if gpu["q"].shape[0] == cfg.T else gpu["q"]
    q_ref = ref["q"][tok]     # the query step covers every token (BatchNorm statistics)
    if cfg.dtype == "bf16":
        dq_abs = np.abs(q_g - q_ref)
        assert (dq_abs <= P.q_allowed(q_g, q_ref)).all(), "q differs by more than one bf16 ulp + fp32 error"
        assert (dq_abs > 0).mean() < 0.01
        C, Cp = O.decode(inp["C"], cfg.dtype), O.decode(inp["Cp"], cfg.dtype)
        sel = P.lookup_chunks(cfg, q_g, C, Cp, score=score)
    else:
        assert P.row_rel_err(q_g, q_ref).max() <= 1e-5
        sel = ref
    G = gpu["idx"][tok] if gpu["idx"].shape[0] == cfg.T else gpu["idx"]
    w_g = gpu["w"][tok] if gpu["w"].shape[0] == cfg.T else gpu["w"]
    y_g = gpu["y"][tok] if gpu["y"].shape[0] == cfg.T else gpu["y"]
    score_of, exact_set, exact_order = P.judge_selection(cfg, sel, G)
    # weights: softmax of the oracle scores of the GPU's own selection
    w_ref = O.softmax(score_of(G), cfg.temperature)
    assert np.abs(w_g - w_ref).max() <= tol * max(1e-3, float(np.abs(w_ref).max()))
    # y: sum of the GPU-selected rows with those weights (equals the oracle's y wherever the sets agree)
    y_ref = O.gather_sum(G.astype(np.int64), w_ref, inp["V"], cfg.dtype)
    assert P.row_rel_err(y_g, y_ref).max() <= tol
    same = exact_set.all(-1) & (np.sort(ref["rows"], -1) == np.sort(G, -1)).all(-1).all(-1)
    if same.any():
        assert P.row_rel_err(y_g[same], ref["y"][same]).max() <= tol
    return {"exact_set": float(exact_set.mean()), "exact_order": float(exact_order.mean()), "ref": ref, "sel": sel,
            "q": q_g}


def run_gpu_forward(cfg, inp):
    layer = layer_for(cfg)
    dev = upload(inp)
    y, saved = layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"])
    torch.cuda.synchronize()
    return {"q": P.to_f64(saved["q"]), "idx": saved["idx"].cpu().numpy(), "w": saved["w"].cpu().numpy(),
            "y": P.to_f64(y)}, (layer, dev, saved, y)


FWD_CASES = {
    "tiny": pi.CONFIGS["tiny"],
    "small": pi.CONFIGS["small"],
    "bf16_mid": _cfg(T=2048, d=256, heads=2, dq=128, n_keys=256, n_keys2=256, topk=32, d_value=256,
                     dtype="bf16", bn=True, seed=21),
    "ragged": _cfg(T=77, d=40, heads=3, dq=48, n_keys=50, n_keys2=33, topk=32, d_value=40, dtype="bf16",
                   bn=True, seed=22),
    "one_token": _cfg(T=1, d=16, heads=2, dq=16, n_keys=16, n_keys2=16, topk=4, d_value=16, dtype="bf16",
                      bn=False, seed=23),
    "k1": _cfg(T=50, d=32, heads=2, dq=32, n_keys=20, n_keys2=30, topk=1, d_value=24, dtype="f32", bn=True,
               seed=24),
    "tau": _cfg(T=90, d=32, heads=2, dq=32, n_keys=40, n_keys2=40, topk=16, d_value=32, dtype="f32", bn=True,
                seed=25, temperature=0.25),
    "int_ties": _cfg(T=40, d=8, heads=2, dq=8, n_keys=12, n_keys2=9, topk=6, d_value=8, dtype="f32", bn=False,
                     seed=26, x_kind="int", wq_kind="int", key_kind="int", int_range=1),
    # few slots, many tokens: every value row gets hundreds of lookups and every
    # sub-key thousands, so the backward splits them into chunks
    "hot": _cfg(T=6000, d=32, heads=2, dq=32, n_keys=8, n_keys2=8, topk=8, d_value=40, dtype="f32", bn=True,
                seed=27),
    "hot_bf16": _cfg(T=6000, d=64, heads=2, dq=64, n_keys=16, n_keys2=16, topk=16, d_value=64, dtype="bf16",
                     bn=True, seed=28),
    # few tokens, wide halves: the scoring splits each half over 4 blocks
    "split": _cfg(T=100, d=32, heads=1, dq=32, n_keys=256, n_keys2=300, topk=8, d_value=32, dtype="f32", bn=True,
                  seed=29),
}


@pytest.mark.parametrize("name", list(FWD_CASES))
def test_forward_end_to_end(name):
    cfg = FWD_CASES[name]
    note(f"forward {name}: {cfg}")
    inp = pi.make_inputs(cfg)
    gpu, _ = run_gpu_forward(cfg, inp)
    stats = forward_check(cfg, inp, gpu)
    if name == "int_ties":
        assert stats["exact_order"] == 1.0
    elif cfg.dtype == "f32":
        assert stats["exact_set"] > 0.999


@pytest.mark.parametrize("name", ["bf16_mid", "ragged", "small", "tau", "k1", "int_ties"])
def test_forward_fused_merge_gather_matches_the_stages(name):
    """pkm_forward merges and gathers in one launch where k divides 64 (else in two): its idx, w and y
    must equal, bit for bit, the merge and gather stage launches run on the same scoring output."""
    from product_key_memory_pkm_amd import pkm_stage_gather, pkm_stage_merge_softmax, pkm_stage_score_topk
    cfg = FWD_CASES[name]
    note(f"fused merge + gather vs stages {name}")
    inp = pi.make_inputs(cfg)
    _, (layer, dev, saved, y) = run_gpu_forward(cfg, inp)
    T, h, k = cfg.T, cfg.heads, cfg.topk
    ws = layer.workspace(T, False)
    si = torch.empty((T, h, 2, k), dtype=torch.int32, device="cuda")
    ss = torch.empty((T, h, 2, k), dtype=torch.float32, device="cuda")
    pkm_stage_score_topk(layer.handle, T, saved["q"], dev["C"], dev["Cp"], si, ss, ws)
    idx = torch.empty((T, h, k), dtype=torch.int32, device="cuda")
    w = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    pkm_stage_merge_softmax(layer.handle, T, si, ss, idx, w)
    y2 = torch.empty_like(y)
    pkm_stage_gather(layer.handle, T, idx, w, dev["V"], y2)
    torch.cuda.synchronize()
    assert torch.equal(idx, saved["idx"])
    assert torch.equal(w.view(torch.int32), saved["w"].view(torch.int32))
    assert torch.equal(y2.view(torch.int16) if y2.dtype == torch.bfloat16 else y2.view(torch.int32),
                       y.view(torch.int16) if y.dtype == torch.bfloat16 else y.view(torch.int32))


def test_forward_is_deterministic():
    cfg = FWD_CASES["bf16_mid"]
    note("forward determinism")
    inp = pi.make_inputs(cfg)
    a, _ = run_gpu_forward(cfg, inp)
    b, _ = run_gpu_forward(cfg, inp)
    for k in a:
        np.testing.assert_array_equal(a[k], b[k])


# ---------------------------------------------------------------------------
# Monitoring signals of a selection ([Blog] §9.3, §11.2; [PKM-summary] key results)
# ---------------------------------------------------------------------------
DIAG_CASES = [
    # T, heads, k, nk, nk2, zipf
    (100, 2, 8, 16, 24, 0.0),
    (3000, 4, 32, 64, 64, 1.1),       # skewed: hot rows and sub-keys
    (1, 1, 1, 4, 4, 0.0),
    (0, 3, 4, 8, 8, 0.0),             # empty batch: zero counts
    (700, 8, 16, 2048, 2048, 0.0),    # the largest codebooks
]


@pytest.mark.parametrize("T,h,k,nk,nk2,zipf", DIAG_CASES)
def test_diagnostics_stage(T, h, k, nk, nk2, zipf):
    note(f"diagnostics T={T} h={h} k={k} nk={nk}/{nk2} zipf={zipf}")
    if T > 0:
        rows, w = pi.random_selection(T * 5 + 3, T, h, k, nk * nk2, zipf=zipf)
        w = w.copy()
        w[::7, :, -1] = 0.0          # some zero weights: their terms count 0
    else:
        rows = np.zeros((0, h, k), dtype=np.int32)
        w = np.zeros((0, h, k), dtype=np.float32)
    cfg = _cfg(T=max(T, 1), heads=h, dq=16, n_keys=nk, n_keys2=nk2, topk=k, dtype="f32", d=16, d_value=16)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_diagnostics
    hc = torch.full((h, nk), -1, dtype=torch.int32, device="cuda")
    hcp = torch.full((h, nk2), -1, dtype=torch.int32, device="cuda")
    used = torch.full((1 + h,), -1, dtype=torch.int64, device="cuda")
    ent = torch.empty((max(T, 1), h), dtype=torch.float32, device="cuda")
    ent_sum = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    rd = to_dev(rows) if T > 0 else torch.zeros(1, dtype=torch.int32, device="cuda")
    wd = to_dev(w.astype(np.float32)) if T > 0 else torch.zeros(1, dtype=torch.float32, device="cuda")
    pkm_diagnostics(layer.handle, T, rd, wd, hc, hcp, used, ent, ent_sum, layer.workspace(max(T, 1), True))
    torch.cuda.synchronize()
    r_hc, r_hcp, r_used, r_ent = O.diagnostics(rows, w.astype(np.float32).astype(np.float64), nk, nk2)
    np.testing.assert_array_equal(hc.cpu().numpy(), r_hc)
    np.testing.assert_array_equal(hcp.cpu().numpy(), r_hcp)
    np.testing.assert_array_equal(used.cpu().numpy(), r_used)
    got = ent.cpu().numpy()[:T].astype(np.float64)
    assert np.all(np.abs(got - r_ent) <= 1e-5 * np.abs(r_ent) + 1e-6)
    total = float(ent_sum.cpu().item())
    assert abs(total - r_ent.sum()) <= 1e-5 * abs(r_ent.sum()) + 1e-6


# ---------------------------------------------------------------------------
# fp8 value storage ([Blog] §16.3): quantization and the fp8 gather
# ---------------------------------------------------------------------------
from tests.gpu_util import fp8_table  # noqa: E402

QUANT_CASES = [
    # rows, d_value, dtype
    (300, 64, "f32"),
    (257, 1600, "bf16"),
    (40, 16, "bf16"),       # one 16-code vector per row
    (33, 2048, "bf16"),     # 128 vectors per row: 2 per lane
    (70, 1024, "f32"),
]


def _quant_input(rows, dv, dtype, seed):
    V = pi.random_array(seed, 1, (rows, dv), dtype="f32").astype(np.float32)
    V *= np.exp(pi.random_array(seed, 2, (rows, 1), dtype="f32", std=3.0)).astype(np.float32)  # wide row scales
    V[0] = 0.0                                            # zero row
    V[1] = 0.0
    V[1, dv // 2] = -3.5                                  # one non-zero element
    if dv >= 16:                                          # exact ties: row max 448 (factor 1) and midpoints
        V[2] = 0.0
        V[2, 0] = 448.0
        V[2, 1:8] = [1.0625, 1.1875, -2.125, 0.0029296875, 17.0, 208.0, -1.3125]
    V[3] *= np.float32(1e-4)                              # tiny values: subnormal codes
    if dtype == "bf16":
        return torch.from_numpy(V).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return V


@pytest.mark.parametrize("rows,dv,dtype", QUANT_CASES)
def test_quantize_values_bit_exact(rows, dv, dtype):
    note(f"quantize rows={rows} dv={dv} {dtype}")
    V = _quant_input(rows, dv, dtype, 21)
    cfg = _cfg(d_value=dv, dtype=dtype, n_keys=32, n_keys2=32, d=16, dq=32)
    layer = layer_for(cfg, values="fp8")
    from product_key_memory_pkm_amd import pkm_quantize_values
    rb = (dv + 16 + 127) // 128 * 128       # row stride: header and codes in whole 128-byte lines
    out = torch.full((rows * rb,), 0xAB, dtype=torch.uint8, device="cuda")
    pkm_quantize_values(layer.handle, to_dev(V), out)
    torch.cuda.synchronize()
    got = out.cpu().numpy().reshape(rows, rb)
    scale, codes = O.quantize_rows_fp8(V, dtype)
    np.testing.assert_array_equal(got[:, :4].copy().view(np.float32).reshape(-1), scale)
    assert (got[:, 4:16] == 0).all()
    np.testing.assert_array_equal(got[:, 16:16 + dv], codes)
    assert (got[:, 16 + dv:] == 0).all()     # every byte of the row is written


FP8_GATHER_CASES = [
    # T, heads, k, rows, d_value, dtype
    (64, 4, 32, 5000, 1600, "bf16"),
    (37, 3, 5, 100, 32, "f32"),
    (33, 1, 3, 50, 2048, "bf16"),      # 4 vectors per lane
    (70, 4, 32, 4096, 768, "f32"),     # 3 vectors per lane
    # the header and the codes over the lanes: exactly 64 vectors, one past, exactly 128
    (20, 2, 8, 300, 1008, "bf16"),
    (20, 2, 8, 300, 1024, "bf16"),
    (20, 2, 8, 300, 2032, "bf16"),
]


@pytest.mark.parametrize("T,h,k,nrows,dv,dtype", FP8_GATHER_CASES)
def test_gather_fp8_values(T, h, k, nrows, dv, dtype):
    note(f"gather fp8 T={T} h={h} k={k} rows={nrows} dv={dv} {dtype}")
    rows, w = pi.random_selection(T + nrows + 1, T, h, k, nrows)
    V = pi.random_array(7, 3, (nrows, dv), dtype="f32", std=dv ** -0.5)
    scale, codes = O.quantize_rows_fp8(V, "f32")       # the table comes from the oracle
    nk = int(np.ceil(np.sqrt(nrows)))
    cfg = _cfg(heads=h, topk=k, n_keys=max(nk, k), n_keys2=max(nk, k), d_value=dv, dtype=dtype,
               d=16 if dtype == "bf16" else 8, dq=32)
    layer = layer_for(cfg, values="fp8")
    from product_key_memory_pkm_amd import pkm_stage_gather
    y = torch.empty((T, dv), dtype=layer.storage, device="cuda")
    pad = cfg.slots - nrows           # the table holds the layer's |C|*|C'| rows (the lookups use the first nrows)
    table = fp8_table(np.concatenate([scale, np.zeros(pad, np.float32)]),
                      np.concatenate([codes, np.zeros((pad, dv), np.uint8)]))
    pkm_stage_gather(layer.handle, T, to_dev(rows), to_dev(w), torch.from_numpy(table).cuda(), y)
    torch.cuda.synchronize()
    ref = O.gather_sum(rows, w.astype(np.float64), O.dequantize_rows_fp8(scale, codes), O.F64)
    err = P.row_rel_err(P.to_f64(y), ref)
    assert err.max() <= (1e-5 if dtype == "f32" else 8e-3), err.max()


def test_forward_with_fp8_values_end_to_end():
    """A bf16 layer whose value table is stored as fp8 rows: the selection is the storage-value layer's, y the
    weighted sum of the dequantized rows."""
    cfg = FWD_CASES["bf16_mid"]
    note(f"forward fp8 values: {cfg}")
    inp = pi.make_inputs(cfg)
    scale, codes = O.quantize_rows_fp8(inp["V"], cfg.dtype)
    layer = layer_for(cfg, values="fp8")
    dev = upload(inp)
    table = torch.from_numpy(fp8_table(scale, codes)).cuda()
    y, saved = layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], table)
    torch.cuda.synchronize()
    ref = O.forward(cfg, inp)
    idx = saved["idx"].cpu().numpy()
    exact = (np.sort(idx, -1) == np.sort(ref["rows"], -1)).all(-1).all(-1)
    assert exact.mean() > 0.95
    y_ref = O.gather_sum(ref["rows"], ref["w"], O.dequantize_rows_fp8(scale, codes), O.F64)
    err = P.row_rel_err(P.to_f64(y)[exact], y_ref[exact])
    assert err.max() <= 8e-3, err.max()
    # the fp8 table reproduces the storage-value output to within its rounding (E4M3: 2^-4 relative per element)
    y_bf16 = O.gather_sum(ref["rows"], ref["w"], inp["V"], cfg.dtype)
    assert P.row_rel_err(y_ref, y_bf16).max() <= 0.1
