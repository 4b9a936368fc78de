"""GPU parity of the backward steps (a7-a10) against the fp64 CPU oracle.

Stage tests feed both sides the same seeded selections, weights and upstream
gradients; end-to-end tests run the GPU forward + backward and the oracle's on
the same seeded layer.  Rules and tolerances: tests/parity.py.
"""
import numpy as np
import pytest
import torch

import pkm_inputs as pi
from oracle import pkm_oracle as O
from tests import parity as P
from tests.gpu_util import layer_for, note, require_lib, to_dev, upload
from tests.test_gpu_forward import FWD_CASES, forward_check, run_gpu_forward

pytestmark = pytest.mark.gpu

SENTINEL = 0.25


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _cfg(**kw):
    base = dict(T=64, d=16, heads=1, dq=32, n_keys=32, n_keys2=32, topk=8, d_value=64, dtype="f32", bn=False,
                seed=3)
    base.update(kw)
    return pi.custom(**base)


# ---------------------------------------------------------------------------
# a7 (dw) + a8 (sparse dV)
# ---------------------------------------------------------------------------
VG_CASES = [
    # T, heads, k, nk (slots = nk^2), d_value, dtype, zipf, accumulate
    (40, 2, 8, 16, 64, "f32", 0.0, True),
    (300, 4, 32, 64, 512, "f32", 0.0, True),
    (300, 4, 32, 64, 512, "f32", 1.2, False),      # skewed: long runs of one row
    (128, 4, 32, 128, 1600, "bf16", 0.0, True),
    (64, 8, 32, 64, 1024, "bf16", 1.0, True),
    (1, 1, 1, 4, 8, "bf16", 0.0, True),
    (2000, 2, 16, 16, 16, "f32", 0.0, True),       # 256 rows, ~250 lookups per row
    # up to 8192 lookups are grouped by one workgroup; one more takes the multi-launch radix sort
    (256, 2, 16, 32, 64, "f32", 1.2, True),        # 8192 lookups, skewed: long runs
    (257, 2, 16, 32, 64, "f32", 1.2, True),        # 8224 lookups
    (1000, 2, 4, 4, 32, "bf16", 0.0, False),       # 8000 lookups over 16 rows: every row split in chunks
    # the radix passes' block shapes: 4-wave blocks with two sub-tiles each (1.5 M lookups), the ragged
    # tail of a skewed 1.2 M, and 16-wave blocks with two sub-tiles each (5.2 M lookups)
    (12000, 4, 32, 1024, 16, "f32", 0.0, True),
    (12345, 3, 32, 1024, 8, "f32", 0.9, False),
    (40960, 4, 32, 1024, 8, "f32", 0.0, True),
]


@pytest.mark.parametrize("T,h,k,nk,dv,dtype,zipf,acc", VG_CASES)
def test_value_grad_stage(T, h, k, nk, dv, dtype, zipf, acc):
    note(f"value_grad T={T} h={h} k={k} slots={nk * nk} dv={dv} {dtype} zipf={zipf} acc={acc}")
    nrows = nk * nk
    rows, w = pi.random_selection(T * 3 + 1, T, h, k, nrows, zipf=zipf)
    V = pi.random_array(8, 1, (nrows, dv), dtype=dtype, std=0.05)
    dY = pi.random_array(8, 2, (T, dv), dtype=dtype)
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=nk, n_keys2=nk, d_value=dv, dtype=dtype)
    layer = layer_for(cfg, accumulate_dv=acc)
    from product_key_memory_pkm_amd import pkm_stage_value_grad
    outs = []
    for rep in range(2):
        dV = torch.full((nrows, dv), SENTINEL, dtype=torch.float32, device="cuda")
        touched = torch.full((T * h * k,), -1, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
        pkm_stage_value_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), to_dev(V), dV, touched, nt, dw,
                             layer.workspace(T, True))
        torch.cuda.synchronize()
        outs.append((dV.cpu().numpy(), touched.cpu().numpy(), int(nt.item()), dw.cpu().numpy()))
    dV, touched, nt, dw = outs[0]
    # bit-identical on a second run (sorted grouping, no atomics)
    np.testing.assert_array_equal(outs[1][0], dV)
    np.testing.assert_array_equal(outs[1][3], dw)
    uniq = np.unique(rows)
    assert nt == len(uniq)
    np.testing.assert_array_equal(touched[:nt], uniq)
    untouched = np.setdiff1d(np.arange(nrows), uniq)
    assert (dV[untouched] == SENTINEL).all(), "an untouched row was written"
    ref_dw = O.weight_grad(rows, dY, V, dtype)
    tol = P.TOL["f32"]
    assert P.row_rel_err(dw.reshape(T, -1), ref_dw.reshape(T, -1)).max() <= (tol if dtype == "f32" else 1e-5)
    ref_dv = O.value_grad_rows(rows, w.astype(np.float64), dY, dtype, uniq)
    got = dV[uniq].astype(np.float64) - (SENTINEL if acc else 0.0)
    sent_ulp = 2.0 ** -24 * SENTINEL if acc else 0.0
    err = np.abs(got - ref_dv).max(1)
    assert (err <= 1e-5 * np.abs(ref_dv).max(1) + 2 * sent_ulp).all()


def test_value_grad_run_length_edges():
    """Rows looked up exactly 1, 255, 256, 257, 512, 513 and 3000 times.

    Runs longer than the kernel's chunk are split over several waves and their
    partial sums combined in order; the lengths straddle the chunk boundaries.
    """
    T, h, k, dv, nrows = 600, 2, 8, 96, 64
    lens = [1, 255, 256, 257, 512, 513, 3000]
    n = T * h * k
    g = np.random.Generator(np.random.PCG64(77))
    fixed = np.concatenate([np.full(c, r, np.int64) for r, c in enumerate(lens)])
    rest = g.integers(len(lens), nrows, size=n - fixed.size)
    rows = g.permutation(np.concatenate([fixed, rest])).astype(np.int32).reshape(T, h, k)
    _, w = pi.random_selection(5, T, h, k, nrows)
    V = pi.random_array(12, 1, (nrows, dv), std=0.05)
    dY = pi.random_array(12, 2, (T, dv))
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=8, n_keys2=8, d_value=dv)
    note(f"value_grad run-length edges {lens}")
    from product_key_memory_pkm_amd import pkm_stage_value_grad
    layer = layer_for(cfg, accumulate_dv=True)
    dV = torch.full((nrows, dv), SENTINEL, dtype=torch.float32, device="cuda")
    touched = torch.full((n,), -1, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    pkm_stage_value_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), to_dev(V), dV, touched, nt, dw,
                         layer.workspace(T, True))
    torch.cuda.synchronize()
    counts = np.bincount(rows.reshape(-1), minlength=nrows)
    assert list(counts[:len(lens)]) == lens
    uniq = np.unique(rows)
    assert int(nt.item()) == len(uniq)
    ref_dv = O.value_grad_rows(rows, w.astype(np.float64), dY, "f32", uniq)
    got = dV.cpu().double().numpy()[uniq] - SENTINEL
    err = np.abs(got - ref_dv).max(1)
    assert (err <= 1e-5 * np.abs(ref_dv).max(1) + 2 * 2.0 ** -24 * SENTINEL).all()
    ref_dw = O.weight_grad(rows, dY, V, "f32")
    assert P.row_rel_err(dw.cpu().numpy().reshape(T, -1), ref_dw.reshape(T, -1)).max() <= 1e-5


# ---------------------------------------------------------------------------
# a7 (softmax backward) + a9 (query and sub-key gradients)
# ---------------------------------------------------------------------------
SK_CASES = [
    # T, heads, dq, nk, nk2, k, dtype, tau
    (50, 2, 32, 16, 24, 8, "f32", 1.0),
    (400, 4, 256, 256, 256, 32, "f32", 1.0),
    (300, 4, 512, 1024, 1024, 32, "bf16", 1.0),
    (77, 3, 16, 9, 40, 9, "bf16", 0.5),
    (4000, 1, 64, 32, 64, 32, "f32", 1.0),     # first-half sub-keys: ~2550 entries each (split runs)
]


@pytest.mark.parametrize("T,h,dq,nk,nk2,k,dtype,tau", SK_CASES)
def test_subkey_grad_stage(T, h, dq, nk, nk2, k, dtype, tau):
    note(f"subkey_grad T={T} h={h} dq={dq} nk={nk}/{nk2} k={k} {dtype}")
    cfg = _cfg(T=T, heads=h, dq=dq, n_keys=nk, n_keys2=nk2, topk=k, dtype=dtype, temperature=tau)
    rows, w = pi.random_selection(T + 5, T, h, k, nk * nk2)
    dw = pi.random_array(9, 3, (T, h, k))
    q = pi.random_array(9, 4, (T, h * dq), dtype=dtype)
    C = pi.random_array(9, 5, (h, nk, dq // 2), dtype=dtype, std=0.1)
    Cp = pi.random_array(9, 6, (h, nk2, dq // 2), dtype=dtype, std=0.1)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_subkey_grad
    dq_g = torch.empty((T, h * dq), dtype=torch.float32, device="cuda")
    dC = torch.full((h, nk, dq // 2), 3.0, dtype=torch.float32, device="cuda")
    dCp = torch.full((h, nk2, dq // 2), 3.0, dtype=torch.float32, device="cuda")
    pkm_stage_subkey_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dw), to_dev(q), to_dev(C), to_dev(Cp),
                          dq_g, dC, dCp, layer.workspace(T, True))
    torch.cuda.synchronize()
    ds = O.softmax_backward(w.astype(np.float64), dw.astype(np.float64), tau)
    ref_dq, ref_dC, ref_dCp = O.subkey_backward(cfg, rows.astype(np.int64), ds, O.decode(q, dtype),
                                                O.decode(C, dtype), O.decode(Cp, dtype))
    assert P.row_rel_err(dq_g.cpu().double().numpy(), ref_dq).max() <= 1e-5
    for got, ref in ((dC, ref_dC), (dCp, ref_dCp)):
        g = got.cpu().double().numpy()
        assert P.fro_rel_err(g, ref) <= 1e-5
        assert (g[np.abs(ref).sum(-1) == 0] == 0).all()     # never-selected sub-keys: exactly zero


# ---------------------------------------------------------------------------
# a10: BatchNorm backward and the projection gradients
# ---------------------------------------------------------------------------
QG_CASES = [
    # T, d, heads, dq, dtype, bn
    (64, 64, 1, 32, "f32", False),
    (500, 128, 2, 64, "f32", True),
    (1000, 1600, 4, 512, "bf16", True),
    (37, 24, 3, 16, "bf16", True),
]


@pytest.mark.parametrize("T,d,h,dq,dtype,bn", QG_CASES)
def test_query_grad_stage(T, d, h, dq, dtype, bn):
    note(f"query_grad T={T} d={d} h={h} dq={dq} {dtype} bn={bn}")
    cfg = _cfg(T=T, d=d, heads=h, dq=dq, dtype=dtype, bn=bn, n_keys=8, n_keys2=8, topk=4, d_value=16, seed=T + 1)
    inp = pi.make_inputs(cfg)
    F = cfg.F
    gamma = np.linspace(0.5, 1.5, F).astype(np.float32)
    dq_in = pi.random_array(10, 0, (T, F), std=0.1)
    # saved state as the forward would leave it: q_pre, batch mean and 1/sqrt(var+eps), all fp32
    ref = O.query(cfg, dict(inp, gamma=gamma))
    q_pre32 = ref["q_pre"].astype(np.float32)
    if bn:
        mean32 = q_pre32.astype(np.float64).mean(0).astype(np.float32)
        var = ((q_pre32.astype(np.float64) - mean32) ** 2).mean(0)
        rstd32 = (1.0 / np.sqrt(var + cfg.bn_eps)).astype(np.float32)
    layer = layer_for(cfg)
    saved = layer.alloc_saved(T)
    saved["q_pre"].copy_(torch.from_numpy(q_pre32))
    if bn:
        saved["bn_mean"].copy_(torch.from_numpy(mean32))
        saved["bn_rstd"].copy_(torch.from_numpy(rstd32))
    dev = upload(inp)
    dWq = torch.empty((F, d), dtype=torch.float32, device="cuda")
    dgamma = torch.empty(F, dtype=torch.float32, device="cuda") if bn else None
    dbeta = torch.empty(F, dtype=torch.float32, device="cuda") if bn else None
    dx = torch.empty((T, d), dtype=layer.storage, device="cuda")
    from product_key_memory_pkm_amd import pkm_stage_query_grad
    pkm_stage_query_grad(layer.handle, T, to_dev(dq_in), dev["x"], dev["Wq"], to_dev(gamma), saved, dWq, dgamma, dbeta,
                         dx, layer.workspace(T, True))
    torch.cuda.synchronize()
    dq64 = dq_in.astype(np.float64)
    if bn:
        xhat = (q_pre32.astype(np.float64) - mean32) * rstd32.astype(np.float64)
        var_eff = 1.0 / rstd32.astype(np.float64) ** 2 - cfg.bn_eps
        dq_pre, dg, db = O.batchnorm_backward(dq64, xhat, gamma.astype(np.float64), var_eff, cfg.bn_eps)
        assert P.fro_rel_err(P.to_f64(dgamma), dg) <= 1e-5
        assert P.fro_rel_err(P.to_f64(dbeta), db) <= 1e-5
    else:
        dq_pre = dq64
    x = O.decode(inp["x"], dtype)
    Wq = O.decode(inp["Wq"], dtype)
    # bf16 storage: dq_pre enters the MFMA products as bf16 (2^-9 relative per element)
    tol = 1e-5 if dtype == "f32" else 1e-2
    assert P.fro_rel_err(P.to_f64(dWq), dq_pre.T @ x) <= tol
    assert P.fro_rel_err(P.to_f64(dx), dq_pre @ Wq) <= tol


# ---------------------------------------------------------------------------
# whole backward
# ---------------------------------------------------------------------------
def reference_forward(cfg, inp, gpu):
    """The oracle's forward on the GPU's selection, after judging it (tests/parity.py: forced_forward).

    Near-tie tokens may validly select other rows than the oracle; with their selection forced on the
    oracle, every gradient has one correct answer and the whole upstream gradient is compared."""
    stats = forward_check(cfg, inp, gpu)
    return P.forced_forward(cfg, stats["ref"], stats["sel"], stats["q"], gpu["idx"]), stats


def backward_check(cfg, inp, gpu, g, dV_np, dY, fwd):
    """Compare a GPU backward with the oracle's for the same upstream gradient dY on the forward ``fwd``."""
    gb = O.backward(cfg, inp, fwd, dY)
    tol = P.TOL[cfg.dtype]
    uniq = np.unique(gpu["idx"])
    nt = int(g["n_touched"].item())
    assert nt == len(uniq)
    np.testing.assert_array_equal(g["touched"].cpu().numpy()[:nt], uniq)
    untouched = np.setdiff1d(np.arange(cfg.slots), uniq)
    assert (dV_np[untouched] == SENTINEL).all()
    rows = uniq
    ref_dv = O.value_grad_rows(fwd["rows"], fwd["w"], dY, cfg.dtype, rows)
    # a row sums w*dY over its lookups; the weights carry the forward's relative error, so the
    # bound is relative to the sum of |w*dY| (rows whose terms cancel would otherwise be held
    # to far less than the inputs' own accuracy)
    dY_abs = (dY & np.uint16(0x7FFF)) if cfg.dtype == "bf16" else np.abs(dY)
    mag = O.value_grad_rows(fwd["rows"], fwd["w"], dY_abs, cfg.dtype, rows)
    got = dV_np[rows].astype(np.float64) - SENTINEL
    err = np.abs(got - ref_dv).max(1)
    assert (err <= tol * mag.max(1) + 2.0 ** -23 * (SENTINEL + np.abs(got).max(1))).all()
    assert P.fro_rel_err(P.to_f64(g["dC"]), gb["dC"]) <= tol
    assert P.fro_rel_err(P.to_f64(g["dCp"]), gb["dCp"]) <= tol
    assert P.fro_rel_err(P.to_f64(g["dWq"]), gb["dWq"]) <= tol
    if cfg.bn:
        assert P.fro_rel_err(P.to_f64(g["dgamma"]), gb["dgamma"]) <= tol
        assert P.fro_rel_err(P.to_f64(g["dbeta"]), gb["dbeta"]) <= tol
    if g.get("dx") is not None:
        assert P.fro_rel_err(P.to_f64(g["dx"]), gb["dx"]) <= tol


BWD_CASES = ["tiny", "small", "bf16_mid", "ragged", "one_token", "k1", "tau", "int_ties", "hot", "hot_bf16"]


@pytest.mark.parametrize("name", BWD_CASES)
def test_backward_end_to_end(name):
    cfg = FWD_CASES[name]
    note(f"backward {name}: {cfg}")
    inp = pi.make_inputs(cfg, with_dy=True)
    gpu, (layer, dev, saved, y) = run_gpu_forward(cfg, inp)
    fwd, _ = reference_forward(cfg, inp, gpu)
    dY = inp["dY"]
    dV = torch.full((cfg.slots, cfg.d_value), SENTINEL, dtype=torch.float32, device="cuda")
    g = layer.backward(to_dev(dY), dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], dev["V"], saved, dV)
    torch.cuda.synchronize()
    backward_check(cfg, inp, gpu, g, dV.cpu().numpy(), dY, fwd)


def test_backward_is_deterministic():
    cfg = FWD_CASES["bf16_mid"]
    note("backward determinism")
    inp = pi.make_inputs(cfg, with_dy=True)
    res = []
    for _ in range(2):
        gpu, (layer, dev, saved, y) = run_gpu_forward(cfg, inp)
        dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
        g = layer.backward(to_dev(inp["dY"]), dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], dev["V"],
                           saved, dV)
        torch.cuda.synchronize()
        out = {k: v.cpu().clone() for k, v in g.items() if v is not None}
        out["touched"] = out["touched"][: int(out["n_touched"].item())]
        out["dV"] = dV.cpu()
        res.append(out)
    for k in res[0]:
        assert torch.equal(res[0][k], res[1][k]), k


def test_row_groups_then_grouped_value_grad_equals_value_grad_stage():
    note("row groups + grouped value grad")
    T, h, k, nk, dv = 300, 4, 32, 64, 1024
    rows, w = pi.random_selection(77, T, h, k, nk * nk)
    V = pi.random_array(8, 1, (nk * nk, dv), dtype="bf16", std=0.05)
    dY = pi.random_array(8, 2, (T, dv), dtype="bf16")
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=nk, n_keys2=nk, d_value=dv, dtype="bf16")
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_row_groups, pkm_stage_value_grad, pkm_stage_value_grad_grouped
    outs = []
    for split in (False, True):
        dV = torch.full((nk * nk, dv), SENTINEL, dtype=torch.float32, device="cuda")
        touched = torch.empty(T * h * k, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
        ws = layer.workspace(T, True)
        if split:
            pkm_stage_row_groups(layer.handle, T, to_dev(rows), touched, nt, ws)
            pkm_stage_value_grad_grouped(layer.handle, T, to_dev(w), to_dev(dY), to_dev(V), dV, dw, nt, ws)
        else:
            pkm_stage_value_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), to_dev(V), dV, touched, nt, dw,
                                 ws)
        torch.cuda.synchronize()
        n = int(nt.item())
        outs.append((dV.cpu(), touched.cpu()[:n], dw.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


# ---------------------------------------------------------------------------
# Adam step on the touched value rows, fused into a8 ([Blog] §6.3)
# ---------------------------------------------------------------------------
ADAM = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, step=5)


def _adam_state(nrows, dv, seed):
    """Moments as after a few earlier steps: m ~ N(0, 1e-3), v ~ U(1e-5, 1e-4)."""
    m0 = pi.random_array(seed, 1, (nrows, dv), dtype="f32", std=1e-3).astype(np.float32)
    v0 = (1e-5 + 9e-5 * np.abs(pi.random_array(seed, 2, (nrows, dv), dtype="f32", std=0.5))).astype(np.float32)
    v0 = np.minimum(v0, np.float32(1e-4))
    return m0, v0


def adam_check(dtype, V0, m0, v0, uniq, g_ref, V1, m1, v1, untouched=None):
    """Rows ``uniq`` against the oracle's Adam step with gradient ``g_ref``; the rows ``untouched`` (default: all
    others) bit-identical to the input."""
    # the boundary carries the hyper-parameters as fp32 (pkm_adam): the oracle gets those values
    hp = {k: (float(np.float32(v)) if k != "step" else v) for k, v in ADAM.items()}
    Vr, mr, vr = O.sparse_adam_rows(V0[uniq], m0[uniq], v0[uniq], g_ref, hp["lr"], hp["beta1"], hp["beta2"],
                                    hp["eps"], hp["step"], dtype)
    nrows = V0.shape[0]
    if untouched is None:
        untouched = np.setdiff1d(np.arange(nrows), uniq)
    np.testing.assert_array_equal(V1[untouched], V0[untouched])
    np.testing.assert_array_equal(m1[untouched], m0[untouched])
    np.testing.assert_array_equal(v1[untouched], v0[untouched])
    gm, gv = m1[uniq].astype(np.float64), v1[uniq].astype(np.float64)
    assert (np.abs(gm - mr).max(1) <= 1e-5 * np.abs(mr).max(1) + 1e-12).all(), "adam m"
    assert (np.abs(gv - vr).max(1) <= 1e-5 * np.abs(vr).max(1) + 1e-15).all(), "adam v"
    gV = O.decode(V1[uniq], dtype)
    err = np.abs(gV - Vr)
    if dtype == "bf16":
        # both sides round to bf16; they may land one bf16 step apart
        assert (err <= P.bf16_ulp(Vr)).all(), "adam V (bf16)"
    else:
        assert (err <= 2.0 ** -22 * np.abs(Vr) + 1e-4 * hp["lr"]).all(), "adam V (f32)"


ADAM_CASES = [
    # T, heads, k, nk (slots = nk^2), d_value, dtype, zipf
    (40, 2, 8, 16, 64, "f32", 0.0),
    (300, 4, 32, 64, 512, "f32", 1.2),       # long runs: chunks, update in the combine launch
    (128, 4, 32, 128, 1600, "bf16", 0.0),
    (64, 8, 32, 64, 1024, "bf16", 1.0),
    (2000, 2, 16, 16, 16, "f32", 0.0),       # ~250 lookups per row, around the chunk size
    (1, 1, 1, 4, 8, "bf16", 0.0),
    (1000, 2, 4, 4, 32, "f32", 0.0),         # one-workgroup grouping, every row split in chunks
]


@pytest.mark.parametrize("T,h,k,nk,dv,dtype,zipf", ADAM_CASES)
def test_value_adam_stage(T, h, k, nk, dv, dtype, zipf):
    note(f"value_adam T={T} h={h} k={k} slots={nk * nk} dv={dv} {dtype} zipf={zipf}")
    nrows = nk * nk
    rows, w = pi.random_selection(T * 3 + 1, T, h, k, nrows, zipf=zipf)
    V = pi.random_array(8, 1, (nrows, dv), dtype=dtype, std=0.05)
    dY = pi.random_array(8, 2, (T, dv), dtype=dtype)
    m0, v0 = _adam_state(nrows, dv, 9)
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=nk, n_keys2=nk, d_value=dv, dtype=dtype)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_value_adam
    outs = []
    for rep in range(2):
        Vd, md, vd = to_dev(V), to_dev(m0), to_dev(v0)
        touched = torch.full((T * h * k,), -1, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
        pkm_stage_value_adam(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), Vd, md, vd, ADAM, touched, nt, dw,
                             layer.workspace(T, True))
        torch.cuda.synchronize()
        Vh = Vd.cpu().view(torch.int16).numpy().view(np.uint16) if dtype == "bf16" else Vd.cpu().numpy()
        outs.append((Vh, md.cpu().numpy(), vd.cpu().numpy(), touched.cpu().numpy(), int(nt.item()),
                     dw.cpu().numpy()))
    V1, m1, v1, touched, nt, dw = outs[0]
    for a, b in zip(outs[0], outs[1]):    # bit-identical from run to run
        np.testing.assert_array_equal(np.asarray(a), np.asarray(b))
    uniq = np.unique(rows)
    assert nt == len(uniq)
    np.testing.assert_array_equal(touched[:nt], uniq)
    # dw comes from the rows before the step
    ref_dw = O.weight_grad(rows, dY, V, dtype)
    assert P.row_rel_err(dw.reshape(T, -1), ref_dw.reshape(T, -1)).max() <= 1e-5
    g_ref = O.value_grad_rows(rows, w.astype(np.float64), dY, dtype, uniq)
    adam_check(dtype, V, m0, v0, uniq, g_ref, V1, m1, v1)


def test_row_groups_then_grouped_adam_equals_adam_stage():
    note("row groups + grouped adam")
    T, h, k, nk, dv = 300, 4, 32, 64, 1024
    rows, w = pi.random_selection(78, T, h, k, nk * nk, zipf=1.2)
    V = pi.random_array(8, 1, (nk * nk, dv), dtype="bf16", std=0.05)
    dY = pi.random_array(8, 2, (T, dv), dtype="bf16")
    m0, v0 = _adam_state(nk * nk, dv, 11)
    cfg = _cfg(T=T, heads=h, topk=k, n_keys=nk, n_keys2=nk, d_value=dv, dtype="bf16")
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_row_groups, pkm_stage_value_adam, pkm_stage_value_adam_grouped
    outs = []
    for split in (False, True):
        Vd, md, vd = to_dev(V), to_dev(m0), to_dev(v0)
        touched = torch.empty(T * h * k, dtype=torch.int32, device="cuda")
        nt = torch.zeros(1, dtype=torch.int64, device="cuda")
        dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
        ws = layer.workspace(T, True)
        if split:
            pkm_stage_row_groups(layer.handle, T, to_dev(rows), touched, nt, ws)
            pkm_stage_value_adam_grouped(layer.handle, T, to_dev(w), to_dev(dY), Vd, md, vd, ADAM, dw, nt, ws)
        else:
            pkm_stage_value_adam(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), Vd, md, vd, ADAM, touched, nt,
                                 dw, ws)
        torch.cuda.synchronize()
        n = int(nt.item())
        outs.append((Vd.cpu(), md.cpu(), vd.cpu(), touched.cpu()[:n], dw.cpu()))
    for a, b in zip(*outs):
        assert torch.equal(a, b)


@pytest.mark.parametrize("name", ["small", "hot"])
def test_backward_adam_end_to_end(name):
    """pkm_backward_adam: the Adam step on the oracle's touched rows, and every other output bit-identical
    to pkm_backward's on the same inputs."""
    cfg = FWD_CASES[name]
    note(f"backward_adam {name}: {cfg}")
    inp = pi.make_inputs(cfg, with_dy=True)
    gpu, (layer, dev, saved, y) = run_gpu_forward(cfg, inp)
    fwd, _ = reference_forward(cfg, inp, gpu)
    dY = inp["dY"]
    dYd = to_dev(dY)
    dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    g_plain = layer.backward(dYd, dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], dev["V"], saved, dV)
    torch.cuda.synchronize()
    plain = {k: v.cpu().clone() for k, v in g_plain.items() if v is not None}
    m0, v0 = _adam_state(cfg.slots, cfg.d_value, 10)
    V0 = inp["V"]
    Vd, md, vd = to_dev(V0), to_dev(m0), to_dev(v0)
    g_adam = layer.backward_adam(dYd, dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], Vd, saved, md, vd,
                                 ADAM)
    torch.cuda.synchronize()
    n = int(plain["n_touched"].item())
    assert int(g_adam["n_touched"].item()) == n
    for k, v in plain.items():
        got = g_adam[k].cpu()
        if k == "touched":
            assert torch.equal(got[:n], v[:n])
        else:
            assert torch.equal(got, v), k
    # the oracle's Adam step on the rows of the (judged) GPU selection, every other row bit-identical
    uniq = np.unique(fwd["rows"])
    untouched = np.setdiff1d(np.arange(cfg.slots), uniq)
    g_ref = O.value_grad_rows(fwd["rows"], fwd["w"], dY, cfg.dtype, uniq)
    Vh = Vd.cpu().view(torch.int16).numpy().view(np.uint16) if cfg.dtype == "bf16" else Vd.cpu().numpy()
    adam_check(cfg.dtype, V0, m0, v0, uniq, g_ref, Vh, md.cpu().numpy(), vd.cpu().numpy(), untouched)
