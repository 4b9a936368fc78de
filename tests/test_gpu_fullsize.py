"""GPU parity at the full workload sizes (paper scale and the skewed workload).

Same kernels and launch shapes as bench.py, for the lookup's steps and for the
fp8 value rows, the fused Adam step and the monitoring signals.  The oracle computes sampled
outputs one by one (BatchNorm statistics always over every token); properties
that hold at any size cover the rest: touched rows equal the distinct selected
rows bit for bit, untouched dV rows keep their sentinel, and the value gradient
conserves sum_r dV[r] = sum over lookups of w * dY[t].
"""
import numpy as np
import pytest
import torch

import pkm_inputs as pi
from oracle import pkm_oracle as O
from tests import parity as P
from tests.gpu_util import layer_for, note, require_lib, to_dev, upload
from tests.test_gpu_forward import forward_check

pytestmark = pytest.mark.gpu

SENTINEL = 0.25


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


_INPUTS = {}


def _inputs(name):
    """Seeded inputs of a named workload (with dY), generated once per module."""
    if name not in _INPUTS:
        _INPUTS[name] = pi.make_inputs(pi.CONFIGS[name], with_dy=True)
    return _INPUTS[name]


def _sample(n, count, seed):
    g = np.random.Generator(np.random.PCG64(seed))
    return np.sort(g.choice(n, size=min(n, count), replace=False))


@pytest.mark.parametrize("name", ["paper", "skewed"])
def test_forward_full_size_sampled(name):
    cfg = pi.CONFIGS[name]
    note(f"full-size forward {name}")
    inp = _inputs(name)
    layer = layer_for(cfg)
    dev = upload({k: inp[k] for k in ('x', 'Wq', 'gamma', 'beta', 'C', 'Cp', 'V')})
    y, saved = layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"])
    torch.cuda.synchronize()
    tok = _sample(cfg.T, 192, 5)
    tk = torch.from_numpy(tok).cuda()
    gpu = {"q": P.to_f64(saved["q"][tk]), "idx": saved["idx"][tk].cpu().numpy(), "w": saved["w"][tk].cpu().numpy(),
           "y": P.to_f64(y[tk])}
    del dev
    stats = forward_check(cfg, inp, gpu, tokens=tok)
    assert stats["exact_set"] > 0.95
    # BatchNorm statistics over all tokens
    ref_q = O.query(cfg, inp)
    np.testing.assert_allclose(saved["bn_mean"].cpu().double().numpy(), ref_q["mean"], rtol=1e-4,
                               atol=1e-5 * np.abs(ref_q["q_pre"]).max())
    np.testing.assert_allclose(saved["bn_rstd"].cpu().double().numpy(), 1 / np.sqrt(ref_q["var"] + cfg.bn_eps),
                               rtol=1e-4)


# The paper workload is checked over every token.  The skewed one (4x the oracle's work) is checked on
# 4096 sampled tokens: every other token gets a zero upstream gradient, so it adds exactly nothing to any
# gradient on either side, and the value rows only it selects must keep their sentinel bits.
E2E_SAMPLE = {"paper": None, "skewed": 4096}


def e2e_upstream(cfg, inp, n_sample):
    """(gradient-carrying tokens, upstream gradient): every token, or ``n_sample`` of them with the other
    tokens' rows of dY set to zero."""
    if n_sample is None:
        return np.arange(cfg.T), inp["dY"]
    tok = _sample(cfg.T, n_sample, 23)
    dY = np.zeros_like(inp["dY"])
    dY[tok] = inp["dY"][tok]
    return tok, dY


def e2e_check(cfg, inp, tok, dY, saved, y, dV, g):
    """A whole forward + backward (saved state, y, dV with SENTINEL in untouched rows, gradients g; torch
    tensors on any device) against the oracle on the gradient-carrying tokens ``tok``."""
    dev = dV.device
    G = saved["idx"].cpu().numpy()
    w_g = saved["w"].cpu().numpy()
    q_g = P.to_f64(saved["q"])
    # the query: the oracle's own projection and BatchNorm over every token, equal or one bf16 ulp apart
    ref = O.query(cfg, inp)
    ref["tokens"] = np.arange(cfg.T)
    dq_abs = np.abs(q_g - ref["q"])
    assert (dq_abs <= P.q_allowed(q_g, ref["q"])).all()
    assert (dq_abs > 0).mean() < 0.01
    # the selection: judged against the oracle's exact search on the GPU's query (no slack)
    C, Cp = O.decode(inp["C"], cfg.dtype), O.decode(inp["Cp"], cfg.dtype)
    sel = P.lookup_chunks(cfg, q_g[tok], C, Cp)
    score_of, exact_set, _ = P.judge_selection(cfg, sel, G[tok])
    assert exact_set.mean() > 0.97
    s_G = score_of(G[tok])
    del sel
    w_ref = O.softmax(s_G, cfg.temperature)
    tol = P.TOL[cfg.dtype]
    assert np.abs(w_g[tok] - w_ref).max() <= tol * float(np.abs(w_ref).max())
    fwd = dict(ref, q=q_g[tok], rows=G[tok].astype(np.int64), scores=s_G, w=w_ref)
    # y on sampled tokens
    ty = _sample(len(tok), 384, 29)
    y_g = P.to_f64(y[torch.from_numpy(tok[ty]).to(y.device)])
    y_ref = O.gather_sum(fwd["rows"][ty], w_ref[ty], inp["V"], cfg.dtype)
    assert P.row_rel_err(y_g, y_ref).max() <= tol

    # dV: the touched rows bit for bit, rows without gradient keep the sentinel, sampled rows with all their
    # lookups
    uniq = np.unique(G)
    n = int(g["n_touched"].item())
    assert n == len(uniq)
    np.testing.assert_array_equal(g["touched"][:n].cpu().numpy(), uniq)
    live = np.unique(G[tok])                  # rows with a lookup of a gradient-carrying token
    mask = torch.ones(cfg.slots, dtype=torch.bool, device=dev)
    mask[torch.from_numpy(live).to(dev).long()] = False
    for lo, hi in _row_chunks(cfg.slots):
        blk, m = dV[lo:hi], mask[lo:hi]
        assert bool((blk[m] == SENTINEL).all().item()), f"a row without gradient changed in [{lo}, {hi})"
    which = live[_sample(len(live), 400, 31)]
    dYt = dY[tok]
    ref_dv = O.value_grad_rows(fwd["rows"], w_ref, dYt, cfg.dtype, which)
    dYt_abs = (dYt & np.uint16(0x7FFF)) if cfg.dtype == "bf16" else np.abs(dYt)
    mag = O.value_grad_rows(fwd["rows"], w_ref, dYt_abs, cfg.dtype, which)
    got = dV[torch.from_numpy(which).to(dev).long()].cpu().double().numpy() - SENTINEL
    err = np.abs(got - ref_dv).max(1)
    assert (err <= tol * mag.max(1) + 2.0 ** -23 * (SENTINEL + np.abs(got).max(1))).all()

    # every reduction gradient by norm, against the oracle's backward on the same selection
    gb = P.backward_chunks(cfg, inp, fwd, dY, tokens=None if len(tok) == cfg.T else tok)
    keys = ["dC", "dCp", "dWq", "dx"] + (["dgamma", "dbeta"] if cfg.bn else [])
    for key in keys:
        e = P.fro_rel_err(P.to_f64(g[key]), gb[key])
        assert e <= tol, (key, e)
    return float(exact_set.mean())


@pytest.mark.timeout(900)
@pytest.mark.parametrize("name", ["paper", "skewed"])
def test_forward_backward_end_to_end_full_size(name):
    cfg = pi.CONFIGS[name]
    note(f"full-size forward + backward end to end: {name}")
    inp = _inputs(name)
    tok, dY = e2e_upstream(cfg, inp, E2E_SAMPLE[name])
    layer = layer_for(cfg)
    dev = upload({kk: inp[kk] for kk in ("x", "Wq", "gamma", "beta", "C", "Cp", "V")})
    y, saved = layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"])
    dV = torch.full((cfg.slots, cfg.d_value), SENTINEL, dtype=torch.float32, device="cuda")
    g = layer.backward(to_dev(dY), dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], dev["V"], saved, dV)
    torch.cuda.synchronize()
    del dev
    e2e_check(cfg, inp, tok, dY, saved, y, dV, g)


def _row_chunks(n, step=1 << 18):
    for lo in range(0, n, step):
        yield lo, min(n, lo + step)


# zipf 0.6 over 4.19M rows puts ~15k lookups on the hottest row, about twice
# what the mixture-query workload selects for its hottest row.
@pytest.mark.parametrize("name,zipf", [("paper", 0.0), ("skewed", 0.6)])
def test_value_grad_full_size(name, zipf):
    cfg = pi.CONFIGS[name]
    note(f"full-size value gradient {name} zipf={zipf}")
    T, h, k = cfg.T, cfg.heads, cfg.topk
    rows, w = pi.random_selection(31, T, h, k, cfg.slots, zipf=zipf)
    inp = _inputs(name)
    V, dY = inp["V"], inp["dY"]
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_value_grad
    dV = torch.full((cfg.slots, cfg.d_value), SENTINEL, dtype=torch.float32, device="cuda")
    touched = torch.empty(T * h * k, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    pkm_stage_value_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), to_dev(V), dV, touched, nt, dw,
                         layer.workspace(T, True))
    torch.cuda.synchronize()
    uniq = np.unique(rows)
    n = int(nt.item())
    assert n == len(uniq)
    np.testing.assert_array_equal(touched[:n].cpu().numpy(), uniq)
    # untouched rows keep the sentinel (checked on the device, in row blocks)
    mask = torch.ones(cfg.slots, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(uniq).cuda().long()] = False
    tot = torch.zeros(cfg.d_value, dtype=torch.float64, device="cuda")
    for lo, hi in _row_chunks(cfg.slots):
        blk, m = dV[lo:hi], mask[lo:hi]
        assert bool((blk[m] == SENTINEL).all().item()), f"untouched row written in [{lo}, {hi})"
        tot += (blk[~m].double() - SENTINEL).sum(0)
    # sampled touched rows: every lookup of the row, from the oracle
    which = uniq[_sample(len(uniq), 400, 9)]
    if zipf > 0:   # include the hottest rows
        vals, cnt = np.unique(rows, return_counts=True)
        which = np.union1d(which, vals[np.argsort(-cnt)[:8]])
    ref = O.value_grad_rows(rows, w.astype(np.float64), dY, cfg.dtype, which)
    dY_abs = dY & np.uint16(0x7FFF)
    mag = O.value_grad_rows(rows, w.astype(np.float64), dY_abs, cfg.dtype, which)
    got = dV[torch.from_numpy(which).cuda().long()].cpu().double().numpy() - SENTINEL
    err = np.abs(got - ref).max(1)
    assert (err <= 1e-5 * mag.max(1) + 2.0 ** -23 * (SENTINEL + np.abs(got).max(1))).all()
    # sampled dw
    tok = _sample(T, 128, 11)
    ref_dw = O.weight_grad(rows[tok], dY[tok], V, cfg.dtype)
    assert P.row_rel_err(dw[torch.from_numpy(tok).cuda()].cpu().double().numpy().reshape(len(tok), -1),
                         ref_dw.reshape(len(tok), -1)).max() <= 1e-5
    # conservation over all rows: sum_r (dV[r] - sentinel) = sum_t (sum_{h,s} w) dY[t]
    tot = tot.cpu().numpy()
    wt = w.astype(np.float64).reshape(T, -1).sum(1)
    expect = wt @ O.decode(dY, cfg.dtype)
    assert np.abs(tot - expect).max() <= 1e-3 * np.abs(expect).max() + 1e-3


@pytest.mark.parametrize("name,zipf", [("paper", 0.0), ("skewed", 0.6)])
def test_subkey_grad_full_size_sampled(name, zipf):
    cfg = pi.CONFIGS[name]
    note(f"full-size sub-key gradient {name} zipf={zipf}")
    T, h, k, dq = cfg.T, cfg.heads, cfg.topk, cfg.dq
    rows, w = pi.random_selection(41, T, h, k, cfg.slots, zipf=zipf)
    dw = pi.random_array(41, 3, (T, h, k))
    q = pi.random_array(41, 4, (T, h * dq), dtype="bf16")
    inp = _inputs(name)
    C, Cp = inp["C"], inp["Cp"]
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_subkey_grad
    dq_g = torch.empty((T, h * dq), dtype=torch.float32, device="cuda")
    dC = torch.full(C.shape, 3.0, dtype=torch.float32, device="cuda")
    dCp = torch.full(Cp.shape, 3.0, dtype=torch.float32, device="cuda")
    pkm_stage_subkey_grad(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dw), to_dev(q), to_dev(C), to_dev(Cp),
                          dq_g, dC, dCp, layer.workspace(T, True))
    torch.cuda.synchronize()
    ds = O.softmax_backward(w.astype(np.float64), dw.astype(np.float64), cfg.temperature)
    Cd, Cpd, qd = O.decode(C, "bf16"), O.decode(Cp, "bf16"), O.decode(q, "bf16")
    # dq on sampled tokens
    tok = _sample(T, 256, 13)
    ref_dq, _, _ = O.subkey_backward(cfg, rows[tok].astype(np.int64), ds[tok], qd[tok], Cd, Cpd)
    assert P.row_rel_err(dq_g[torch.from_numpy(tok).cuda()].cpu().double().numpy(), ref_dq).max() <= 1e-5
    # dC / dC' rows of sampled sub-keys: every lookup of that sub-key
    g1, g2 = dC.cpu().double().numpy(), dCp.cpu().double().numpy()
    half = dq // 2
    hh = np.broadcast_to(np.arange(h)[None, :, None], rows.shape)
    for half_sel, G, nk in ((0, g1, cfg.n_keys), (1, g2, cfg.n_keys2)):
        sub = rows // cfg.n_keys2 if half_sel == 0 else rows % cfg.n_keys2
        picks = [(0, 0), (1, 17), (h - 1, nk - 1), (2, nk // 2 - 1), (0, 700)]
        # the most used sub-keys (the longest runs)
        flat = (hh * nk + sub).reshape(-1)
        cnt = np.bincount(flat, minlength=h * nk)
        picks += [(int(f // nk), int(f % nk)) for f in np.argsort(-cnt)[:3]]
        for (h0, i0) in picks:
            sel = (hh == h0) & (sub == i0)
            t_idx = np.nonzero(sel)[0]
            qh = qd.reshape(T, h, 2, half)[t_idx, h0, half_sel, :]
            ref = (ds[sel][:, None] * qh).sum(0)
            got = G[h0, i0]
            scale = (np.abs(ds[sel])[:, None] * np.abs(qh)).sum(0).max() + 1e-30
            assert np.abs(got - ref).max() <= 1e-5 * scale, (half_sel, h0, i0)
    # sub-keys never selected: exactly zero
    used = np.zeros((h, cfg.n_keys), bool)
    used[hh.reshape(-1), (rows // cfg.n_keys2).reshape(-1)] = True
    assert (g1[~used] == 0).all()


def test_query_grad_full_size():
    cfg = pi.CONFIGS["paper"]
    note("full-size query gradient (paper)")
    T, F = cfg.T, cfg.F
    inp = _inputs("paper")
    ref = O.query(cfg, inp)
    q_pre32 = ref["q_pre"].astype(np.float32)
    mean32 = q_pre32.astype(np.float64).mean(0).astype(np.float32)
    var = ((q_pre32.astype(np.float64) - mean32) ** 2).mean(0)
    rstd32 = (1.0 / np.sqrt(var + cfg.bn_eps)).astype(np.float32)
    dq_in = pi.random_array(51, 0, (T, F), std=0.1)
    gamma = np.linspace(0.5, 1.5, F).astype(np.float32)
    layer = layer_for(cfg)
    saved = layer.alloc_saved(T)
    saved["q_pre"].copy_(torch.from_numpy(q_pre32))
    saved["bn_mean"].copy_(torch.from_numpy(mean32))
    saved["bn_rstd"].copy_(torch.from_numpy(rstd32))
    dev = upload({"x": inp["x"], "Wq": inp["Wq"]})
    dWq = torch.empty((F, cfg.d), dtype=torch.float32, device="cuda")
    dg = torch.empty(F, dtype=torch.float32, device="cuda")
    db = torch.empty(F, dtype=torch.float32, device="cuda")
    dx = torch.empty((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    from product_key_memory_pkm_amd import pkm_stage_query_grad
    pkm_stage_query_grad(layer.handle, T, to_dev(dq_in), dev["x"], dev["Wq"], to_dev(gamma), saved, dWq, dg, db, dx,
                         layer.workspace(T, True))
    torch.cuda.synchronize()
    xhat = (q_pre32.astype(np.float64) - mean32) * rstd32.astype(np.float64)
    var_eff = 1.0 / rstd32.astype(np.float64) ** 2 - cfg.bn_eps
    dq_pre, dgr, dbr = O.batchnorm_backward(dq_in.astype(np.float64), xhat, gamma.astype(np.float64), var_eff,
                                            cfg.bn_eps)
    assert P.fro_rel_err(P.to_f64(dg), dgr) <= 1e-5
    assert P.fro_rel_err(P.to_f64(db), dbr) <= 1e-5
    x = O.decode(inp["x"], "bf16")
    assert P.fro_rel_err(P.to_f64(dWq), dq_pre.T @ x) <= 1e-2
    tok = _sample(T, 512, 17)
    Wq = O.decode(inp["Wq"], "bf16")
    assert P.fro_rel_err(P.to_f64(dx[torch.from_numpy(tok).cuda()]), dq_pre[tok] @ Wq) <= 1e-2


# ---------------------------------------------------------------------------
# The NEXT rows at full size: fp8 value rows, the fused Adam step, diagnostics
# ---------------------------------------------------------------------------
def test_fp8_values_full_size_sampled():
    # the paper-scale table quantized on the GPU (bit-exact on sampled rows), then the fp8 gather of a
    # paper-shaped selection on sampled tokens against the oracle's own quantization of their rows
    cfg = pi.CONFIGS["paper"]
    note("full-size fp8 values (paper)")
    inp = _inputs("paper")
    V = inp["V"]
    layer = layer_for(cfg, values="fp8")
    from product_key_memory_pkm_amd import pkm_quantize_values, pkm_stage_gather
    rb = (cfg.d_value + 16 + 127) // 128 * 128   # fp8 row stride
    table = torch.empty(cfg.slots * rb, dtype=torch.uint8, device="cuda")
    pkm_quantize_values(layer.handle, to_dev(V), table)
    torch.cuda.synchronize()
    which = _sample(cfg.slots, 2000, 13)
    got = table.view(cfg.slots, rb)[torch.from_numpy(which).cuda()].cpu().numpy()
    scale, codes = O.quantize_rows_fp8(V[which], cfg.dtype)
    np.testing.assert_array_equal(got[:, :4].copy().view(np.float32).reshape(-1), scale)
    assert (got[:, 4:16] == 0).all()
    np.testing.assert_array_equal(got[:, 16:16 + cfg.d_value], codes)
    assert (got[:, 16 + cfg.d_value:] == 0).all()
    T, h, k = cfg.T, cfg.heads, cfg.topk
    rows, w = pi.random_selection(37, T, h, k, cfg.slots)
    y = torch.empty((T, cfg.d_value), dtype=torch.bfloat16, device="cuda")
    pkm_stage_gather(layer.handle, T, to_dev(rows), to_dev(w), table, y)
    torch.cuda.synchronize()
    tok = _sample(T, 128, 17)
    r = rows[tok]
    uniq, inv = np.unique(r, return_inverse=True)
    s_u, c_u = O.quantize_rows_fp8(V[uniq], cfg.dtype)
    ref = O.gather_sum(inv.reshape(r.shape), w[tok].astype(np.float64), O.dequantize_rows_fp8(s_u, c_u), O.F64)
    err = P.row_rel_err(P.to_f64(y[torch.from_numpy(tok).cuda()]), ref)
    assert err.max() <= 8e-3, err.max()


def test_value_adam_full_size_sampled():
    # the first Adam step (zero moments) of the touched rows of a paper-shaped selection
    cfg = pi.CONFIGS["paper"]
    note("full-size value gradient with the Adam step (paper)")
    T, h, k = cfg.T, cfg.heads, cfg.topk
    rows, w = pi.random_selection(41, T, h, k, cfg.slots)
    inp = _inputs("paper")
    V, dY = inp["V"], inp["dY"]
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_value_adam
    hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, step=1)
    V0 = to_dev(V)
    V1 = V0.clone()
    m = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    v = torch.zeros_like(m)
    touched = torch.empty(T * h * k, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    pkm_stage_value_adam(layer.handle, T, to_dev(rows), to_dev(w), to_dev(dY), V1, m, v, hp, touched, nt, dw,
                         layer.workspace(T, True))
    torch.cuda.synchronize()
    uniq = np.unique(rows)
    assert int(nt.item()) == len(uniq)
    # untouched rows: value bits and zero moments kept (checked on the device, in row blocks)
    mask = torch.ones(cfg.slots, dtype=torch.bool, device="cuda")
    mask[torch.from_numpy(uniq).cuda().long()] = False
    for lo, hi in _row_chunks(cfg.slots):
        mk = mask[lo:hi]
        assert torch.equal(V1[lo:hi][mk].view(torch.int16), V0[lo:hi][mk].view(torch.int16)), f"[{lo}, {hi})"
        assert bool((m[lo:hi][mk] == 0).all().item()) and bool((v[lo:hi][mk] == 0).all().item())
    which = uniq[_sample(len(uniq), 400, 19)]
    g = O.value_grad_rows(rows, w.astype(np.float64), dY, cfg.dtype, which)
    f32 = {kk: (float(np.float32(vv)) if kk != "step" else vv) for kk, vv in hp.items()}
    z = np.zeros((len(which), cfg.d_value), dtype=np.float32)
    Vr, mr, vr = O.sparse_adam_rows(V[which], z, z, g, f32["lr"], f32["beta1"], f32["beta2"], f32["eps"],
                                    f32["step"], cfg.dtype)
    wt = torch.from_numpy(which).cuda().long()
    gm, gv = m[wt].cpu().double().numpy(), v[wt].cpu().double().numpy()
    assert (np.abs(gm - mr).max(1) <= 1e-5 * np.abs(mr).max(1) + 1e-12).all(), "adam m"
    assert (np.abs(gv - vr).max(1) <= 1e-5 * np.abs(vr).max(1) + 1e-15).all(), "adam v"
    assert (np.abs(P.to_f64(V1[wt]) - Vr) <= P.bf16_ulp(Vr)).all(), "adam V (bf16)"



def test_value_adam_rows_full_size_against_dense_moments():
    # two Adam steps of paper-shaped selections (about a million touched rows each) with the moments in pool
    # slots and in dense tables: value tables bit-identical; the first step's slots in ascending row order;
    # pool rows equal to the dense rows they stand for
    cfg = pi.CONFIGS["paper"]
    note("full-size Adam step with moments in pool slots against dense moments (paper)")
    T, h, k = cfg.T, cfg.heads, cfg.topk
    inp = _inputs("paper")
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_stage_value_adam, pkm_stage_value_adam_rows
    Vd = to_dev(inp["V"])
    Vr = Vd.clone()
    dY = to_dev(inp["dY"])
    md = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")
    vd = torch.zeros_like(md)
    st = layer.adam_row_state(cfg.slots)
    touched = torch.empty(T * h * k, dtype=torch.int32, device="cuda")
    nt = torch.zeros(1, dtype=torch.int64, device="cuda")
    dw = torch.empty((T, h, k), dtype=torch.float32, device="cuda")
    ws = layer.workspace(T, True)
    seen = np.zeros(0, dtype=np.int64)
    for step, seed in ((1, 41), (2, 42)):
        rows, w = pi.random_selection(seed, T, h, k, cfg.slots)
        rd, wd = to_dev(rows), to_dev(w)
        hp = dict(lr=1e-2, beta1=0.9, beta2=0.999, eps=1e-8, step=step)
        pkm_stage_value_adam(layer.handle, T, rd, wd, dY, Vd, md, vd, hp, touched, nt, dw, ws)
        pkm_stage_value_adam_rows(layer.handle, T, rd, wd, dY, Vr, st, hp, touched, nt, dw, ws)
        torch.cuda.synchronize()
        uniq = np.unique(rows)
        fresh = np.setdiff1d(uniq, seen)
        seen = np.union1d(seen, uniq)
        for lo, hi in _row_chunks(cfg.slots):
            assert torch.equal(Vd[lo:hi].view(torch.int16), Vr[lo:hi].view(torch.int16)), f"step {step} [{lo}, {hi})"
        slot = st["slot"].cpu().numpy()
        assert int(st["n_used"].item()) == seen.size
        np.testing.assert_array_equal(slot[fresh], np.arange(seen.size - fresh.size, seen.size))
        assert (slot[np.setdiff1d(np.arange(cfg.slots), seen)] == -1).all()
        if step == 1:
            np.testing.assert_array_equal(slot[uniq], np.arange(uniq.size))
        for lo in range(0, seen.size, 1 << 17):
            r = torch.from_numpy(seen[lo:lo + (1 << 17)]).cuda().long()
            sl = st["slot"][r].long()
            assert torch.equal(st["m"][sl], md[r]) and torch.equal(st["v"][sl], vd[r]), f"step {step} moments"


@pytest.mark.parametrize("name,zipf", [("paper", 0.0), ("skewed", 0.8)])
def test_diagnostics_full_size(name, zipf):
    # exact integer counts over the whole selection; entropies within fp32 rounding
    cfg = pi.CONFIGS[name]
    note(f"full-size diagnostics {name} zipf={zipf}")
    T, h, k = cfg.T, cfg.heads, cfg.topk
    rows, w = pi.random_selection(43, T, h, k, cfg.slots, zipf=zipf)
    layer = layer_for(cfg)
    from product_key_memory_pkm_amd import pkm_diagnostics
    hc = torch.full((h, cfg.n_keys), -1, dtype=torch.int32, device="cuda")
    hcp = torch.full((h, cfg.n_keys2), -1, dtype=torch.int32, device="cuda")
    used = torch.full((1 + h,), -1, dtype=torch.int64, device="cuda")
    ent = torch.empty((T, h), dtype=torch.float32, device="cuda")
    ent_sum = torch.full((1,), -1.0, dtype=torch.float64, device="cuda")
    pkm_diagnostics(layer.handle, T, to_dev(rows), to_dev(w), hc, hcp, used, ent, ent_sum, layer.workspace(T, True))
    torch.cuda.synchronize()
    r_hc, r_hcp, r_used, r_ent = O.diagnostics(rows, w.astype(np.float64), cfg.n_keys, cfg.n_keys2)
    np.testing.assert_array_equal(hc.cpu().numpy(), r_hc)
    np.testing.assert_array_equal(hcp.cpu().numpy(), r_hcp)
    np.testing.assert_array_equal(used.cpu().numpy(), r_used)
    got = ent.cpu().numpy().astype(np.float64)
    assert np.all(np.abs(got - r_ent) <= 1e-5 * np.abs(r_ent) + 1e-6)
    assert abs(float(ent_sum.cpu().item()) - r_ent.sum()) <= 1e-5 * abs(r_ent.sum()) + 1e-6
