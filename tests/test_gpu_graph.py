"""Forward + backward captured in a HIP graph (torch.cuda.graph) and replayed.

The library enqueues kernels only (no allocation, no memset nodes) and forks
part of the backward onto its side stream with events, so the whole step can
be captured.  Each replay runs between unrelated eager work and must reproduce
the eager results bit for bit (the kernels are deterministic).
"""
import numpy as np
import pytest
import torch

import pkm_inputs as pi
from tests.gpu_util import layer_for, note, require_lib, to_dev, upload
from tests.test_gpu_forward import FWD_CASES

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


@pytest.mark.parametrize("name", ["bf16_mid", "hot"])
def test_forward_backward_graph_replays(name):
    cfg = FWD_CASES[name]
    note(f"graph capture {name}")
    inp = pi.make_inputs(cfg, with_dy=True)
    layer = layer_for(cfg, accumulate_dv=False)
    dev = upload({k: inp[k] for k in ("x", "Wq", "gamma", "beta", "C", "Cp", "V")})
    dY = to_dev(inp["dY"])
    T = cfg.T
    saved = layer.alloc_saved(T)
    y = torch.empty((T, cfg.d_value), dtype=layer.storage, device="cuda")
    dV = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.float32, device="cuda")

    def step(grads):
        layer.forward(dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"], saved=saved, y=y)
        return layer.backward(dY, dev["x"], dev["Wq"], dev["gamma"], dev["C"], dev["Cp"], dev["V"], saved, dV,
                              out=grads)

    # eager reference (also allocates the workspace and the gradient buffers)
    grads = step(None)
    torch.cuda.synchronize()
    n = int(grads["n_touched"].item())
    touched = grads["touched"][:n].clone()

    def snapshot():
        out = {"y": y.clone(), "idx": saved["idx"].clone(), "w": saved["w"].clone(), "dV": dV[touched.long()].clone()}
        for k_, v_ in grads.items():
            if v_ is not None:
                out[k_] = v_.clone()
        return out

    ref = snapshot()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step(grads)  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        step(grads)
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        for tens in (y, saved["idx"], saved["w"], dV, grads["dC"], grads["dWq"]):
            tens.zero_()
        junk += torch.randn_like(junk)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for k_, v_ in ref.items():
            assert torch.equal(got[k_], v_), f"replay {rep}: {k_} differs from the eager run"


@pytest.mark.parametrize("streams", [1, 8])
def test_fwpkm_chunks_graph_replays(streams):
    # three memorization chunks in sequence (each reads the previous one's write) captured in one graph;
    # one stream groups its 2048 lookups in one workgroup, eight streams take the radix sort
    tps, nchunks, lr = 256, 3, 0.5
    cfg = pi.custom(T=tps * streams, d=16, heads=1, dq=32, n_keys=64, n_keys2=64, topk=8, d_value=64, dtype="bf16",
                    bn=False, seed=52)
    note(f"graph capture of {nchunks} fwpkm chunks, {streams} streams")
    half = cfg.dq // 2
    T = cfg.T
    C = to_dev(pi.random_array(cfg.seed, 1, (1, cfg.n_keys, half), dtype="bf16", std=half ** -0.5))
    Cp = to_dev(pi.random_array(cfg.seed, 2, (1, cfg.n_keys2, half), dtype="bf16", std=half ** -0.5))
    qs = [to_dev(pi.random_array(cfg.seed, 10 + c, (T, cfg.dq), dtype="bf16", std=half ** -0.5)) for c in range(nchunks)]
    ts = [to_dev(pi.random_array(cfg.seed, 20 + c, (T, cfg.d_value), dtype="bf16")) for c in range(nchunks)]
    V0 = to_dev(pi.random_array(cfg.seed, 3, (streams * cfg.slots, cfg.d_value), dtype="bf16", std=0.125))
    layer = layer_for(cfg, score="idw")
    outs = [{"y": torch.empty((T, cfg.d_value), dtype=torch.bfloat16, device="cuda"),
             "idx": torch.empty((T, 1, cfg.topk), dtype=torch.int32, device="cuda"),
             "w": torch.empty((T, 1, cfg.topk), dtype=torch.float32, device="cuda")} for _ in range(nchunks)]
    V = V0.clone()

    def run():
        for c in range(nchunks):
            layer.fwpkm_chunk(qs[c], C, Cp, V, ts[c], lr, out=outs[c], streams=streams)

    def snapshot():
        return [{k_: v_.clone() for k_, v_ in o.items()} for o in outs], V.clone()

    run()  # eager reference (also allocates the workspace)
    torch.cuda.synchronize()
    ref_outs, ref_V = snapshot()
    assert not torch.equal(ref_V, V0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        V.copy_(V0)
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        V.copy_(V0)
        for o in outs:
            for v_ in o.values():
                v_.zero_()
        junk += torch.randn_like(junk)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        got_outs, got_V = snapshot()
        assert torch.equal(got_V, ref_V), f"replay {rep}: the table differs from the eager run"
        for c in range(nchunks):
            for k_ in ("y", "idx", "w"):
                assert torch.equal(got_outs[c][k_], ref_outs[c][k_]), f"replay {rep}: chunk {c} {k_} differs"


@pytest.mark.parametrize("streams", [1, 8])
def test_fwpkm_one_call_graph_replays(streams):
    # three memorization slices in one pkm_fwpkm_chunks call (selection and grouping up front, then the
    # slices' gathers and value steps) captured in one graph and replayed against the eager call
    tps, ncalls, lr = 256, 3, 0.5
    cfg = pi.custom(T=tps * streams, d=16, heads=1, dq=32, n_keys=64, n_keys2=64, topk=8, d_value=64, dtype="bf16",
                    bn=False, seed=54)
    note(f"graph capture of one fwpkm call over {ncalls} slices, {streams} streams")
    half = cfg.dq // 2
    T = cfg.T * ncalls
    C = to_dev(pi.random_array(cfg.seed, 1, (1, cfg.n_keys, half), dtype="bf16", std=half ** -0.5))
    Cp = to_dev(pi.random_array(cfg.seed, 2, (1, cfg.n_keys2, half), dtype="bf16", std=half ** -0.5))
    q = to_dev(pi.random_array(cfg.seed, 10, (T, cfg.dq), dtype="bf16", std=half ** -0.5))
    t = to_dev(pi.random_array(cfg.seed, 20, (T, cfg.d_value), dtype="bf16"))
    V0 = to_dev(pi.random_array(cfg.seed, 3, (streams * cfg.slots, cfg.d_value), dtype="bf16", std=0.125))
    layer = layer_for(cfg, score="idw")
    out = {"y": torch.empty((T, cfg.d_value), dtype=torch.bfloat16, device="cuda"),
           "idx": torch.empty((T, 1, cfg.topk), dtype=torch.int32, device="cuda"),
           "w": torch.empty((T, 1, cfg.topk), dtype=torch.float32, device="cuda")}
    V = V0.clone()

    def run():
        layer.fwpkm_chunks(q, C, Cp, V, t, lr, cfg.T, out=out, streams=streams)

    run()  # eager reference (also allocates the workspace)
    torch.cuda.synchronize()
    ref = {k_: v_.clone() for k_, v_ in out.items()}
    ref_V = V.clone()
    assert not torch.equal(ref_V, V0)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        V.copy_(V0)
        run()  # warm-up on the capture stream
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    junk = torch.zeros(1 << 20, device="cuda")
    for rep in range(3):
        V.copy_(V0)
        for v_ in out.values():
            v_.zero_()
        junk += torch.randn_like(junk)  # unrelated eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(V, ref_V), f"replay {rep}: the table differs from the eager run"
        for k_ in ("y", "idx", "w"):
            assert torch.equal(out[k_], ref[k_]), f"replay {rep}: {k_} differs"
