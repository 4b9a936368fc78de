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
