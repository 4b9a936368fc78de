"""pkm_forward_noalloc (the forward with the library's static per-device scratch as its workspace) against
pkm_forward with a caller workspace: the same kernels on the same inputs, so every output must be bit-identical.
Two calls in a row, the second with fewer tokens (the scratch keeps the first call's contents), at the largest T
the scratch serves for the paper-scale key shape, and at a small fp32 layer."""
import numpy as np
import pytest
import torch

import pkm_inputs as pi
from tests.gpu_util import layer_for, note, require_lib, upload

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = 128 << 20


@pytest.fixture(scope="module", autouse=True)
def _lib():
    require_lib()


def _max_tokens(layer):
    from product_key_memory_pkm_amd import pkm_workspace_size
    c = layer.cfg
    lo, hi = 1, (1 << 26) // (c.heads * c.topk)     # the lookups per call the library takes
    while lo < hi:
        m = (lo + hi + 1) // 2
        if pkm_workspace_size(layer.handle, m, 0) <= SCRATCH_BYTES:
            lo = m
        else:
            hi = m - 1
    return lo


def _both(layer, cfg, inp, T):
    from product_key_memory_pkm_amd import pkm_forward, pkm_forward_noalloc
    dev = upload({k: (v[:T] if k == "x" else v) for k, v in inp.items() if k in ("x", "Wq", "gamma", "beta", "C",
                                                                                  "Cp", "V")})
    outs = []
    for noalloc in (False, True):
        saved = layer.alloc_saved(T)
        for t in saved.values():
            t.fill_(7)                      # every saved buffer must be written by the call
        y = torch.full((T, cfg.d_value), 7, dtype=layer.storage, device="cuda")
        args = (layer.handle, T, dev["x"], dev["Wq"], dev["gamma"], dev["beta"], dev["C"], dev["Cp"], dev["V"], y,
                saved)
        if noalloc:
            pkm_forward_noalloc(*args)
        else:
            pkm_forward(*args, layer.workspace(T, False))
        torch.cuda.synchronize()
        outs.append({"y": y, **saved})
    for k in outs[0]:
        a, b = outs[0][k], outs[1][k]
        assert torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                           b.view(torch.int16) if b.dtype == torch.bfloat16 else b), k


@pytest.mark.parametrize("name", ["paper_keys", "small_f32"])
def test_forward_noalloc_equals_forward(name):
    if name == "paper_keys":
        # the paper-scale key shape (h = 4, dq = 512, 1024 x 1024 slots, k = 32) with narrow rows; the scratch
        # size depends on T and the key shape only
        cfg0 = pi.custom(T=1, d=64, heads=4, dq=512, n_keys=1024, n_keys2=1024, topk=32, d_value=64, dtype="bf16",
                         bn=True, seed=71)
        layer = layer_for(cfg0)
        t_big, t_small = _max_tokens(layer), 3000
    else:
        cfg0 = pi.custom(T=1, d=32, heads=2, dq=32, n_keys=40, n_keys2=36, topk=8, d_value=24, dtype="f32", bn=True,
                         seed=72)
        layer = layer_for(cfg0)
        t_big, t_small = 2048, 77
    cfg = pi.with_tokens(cfg0, t_big)
    inp = pi.make_inputs(cfg)
    for T in (t_big, t_small):
        note(f"forward_noalloc {name} T={T}")
        _both(layer, pi.with_tokens(cfg0, T), inp, T)


def test_forward_noalloc_rejects_tokens_beyond_the_scratch():
    from product_key_memory_pkm_amd import PkmError, pkm_forward_noalloc
    cfg = pi.custom(T=1, d=64, heads=4, dq=512, n_keys=1024, n_keys2=1024, topk=32, d_value=64, dtype="bf16",
                    bn=True, seed=73)
    layer = layer_for(cfg)
    T = _max_tokens(layer) + 1
    note(f"forward_noalloc rejects T={T}")
    x = torch.zeros((T, cfg.d), dtype=torch.bfloat16, device="cuda")
    Wq = torch.zeros((cfg.F, cfg.d), dtype=torch.bfloat16, device="cuda")
    g = torch.ones(cfg.F, device="cuda")
    C = torch.zeros((cfg.heads, cfg.n_keys, cfg.dq // 2), dtype=torch.bfloat16, device="cuda")
    V = torch.zeros((cfg.slots, cfg.d_value), dtype=torch.bfloat16, device="cuda")
    y = torch.empty((T, cfg.d_value), dtype=torch.bfloat16, device="cuda")
    with pytest.raises(PkmError) as e:
        pkm_forward_noalloc(layer.handle, T, x, Wq, g, g, C, C, V, y, layer.alloc_saved(T))
    assert "scratch" in str(e.value)
