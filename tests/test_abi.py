"""The C ABI on the CPU: the library loads, exports what include/pkm.h declares,
and rejects bad arguments before any HIP call.

No test here reaches a kernel launch: every call below fails validation, so the
file is safe with or without a GPU.
"""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "pkm.h")


def _lib():
    from product_key_memory_pkm_amd import _lib as L
    if not os.path.exists(L.LIB_PATH):
        pytest.skip("libpkm.so not built")
    return L


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(pkm_[a-z_0-9]+)\s*\(", src)))


def test_header_declares_the_boundary():
    names = _declared()
    for n in ("pkm_create", "pkm_destroy", "pkm_workspace_size", "pkm_forward", "pkm_backward",
              "pkm_stage_score_topk", "pkm_stage_merge_softmax", "pkm_stage_gather", "pkm_stage_value_grad"):
        assert n in names


def test_library_exports_every_declared_symbol():
    L = _lib()
    lib = L.lib()
    for n in _declared():
        assert hasattr(lib, n), n
    assert sorted(_declared()) == sorted(L.EXPORTED)


def _cfg(L, **kw):
    base = dict(d_in=64, heads=2, d_query=32, n_keys=32, n_keys2=32, topk=8, d_value=64, dtype="f32", bn=True)
    base.update(kw)
    return L.make_config(**base)


BAD_CONFIGS = [
    (dict(d_in=0), 1), (dict(heads=0), 1), (dict(d_query=7), 1), (dict(n_keys=0), 1), (dict(topk=0), 1),
    (dict(topk=40, n_keys=64, n_keys2=64), 2),      # above the 32 the kernels implement
    (dict(topk=16, n_keys=8), 1),                   # k larger than a codebook
    (dict(d_value=0), 1), (dict(temperature=0.0), 1), (dict(temperature=-1.0), 1),
    (dict(n_keys=4096, n_keys2=8), 2),              # codebook above 2048
    (dict(d_in=6), 2), (dict(d_query=6), 2), (dict(d_value=6), 2),   # fp32 needs multiples of 4
    (dict(dtype="bf16", d_in=12), 2), (dict(dtype="bf16", d_query=24), 2),
    (dict(d_value=8192), 2),
    (dict(values="fp8", d_value=40), 2),            # fp8 rows need multiples of 16
]


def test_make_config_rejects_unknown_score():
    L = _lib()
    with pytest.raises(ValueError):
        _cfg(L, score="cosine")


@pytest.mark.parametrize("kw,status", BAD_CONFIGS)
def test_create_rejects(kw, status):
    L = _lib()
    with pytest.raises(L.PkmError) as e:
        L.pkm_create(_cfg(L, **kw))
    assert e.value.status == status


def test_create_row_id_overflow_and_limits():
    L = _lib()
    c = _cfg(L)
    h = L.pkm_create(c)
    got = L.pkm_get_config(h)
    assert (got.d_in, got.heads, got.topk) == (64, 2, 8)
    # unknown enums
    for field, val in (("dtype", 7), ("bn", 5)):
        c2 = _cfg(L)
        setattr(c2, field, val)
        with pytest.raises(L.PkmError):
            L.pkm_create(c2)


def test_workspace_sizes_grow_with_tokens():
    L = _lib()
    h = L.pkm_create(_cfg(L))
    a = L.pkm_workspace_size(h, 100, False)
    b = L.pkm_workspace_size(h, 1000, False)
    c = L.pkm_workspace_size(h, 1000, True)
    assert 0 < a < b <= c
    assert L.pkm_workspace_size(h, 0, True) >= 0
    with pytest.raises(L.PkmError):
        L.pkm_workspace_size(h, -1, False)
    with pytest.raises(L.PkmError) as e:
        L.pkm_workspace_size(h, 1 << 30, False)
    assert e.value.status == L.PKM_ERR_UNSUPPORTED


# Raw calls with fake, 16-byte aligned addresses: validation must fail before they are used.
FAKE = 0x100000


def _fake(n=0):
    return ctypes.c_void_p(FAKE + 256 * n)


def _fwd(L, h, T=10, **over):
    args = dict(x=_fake(1), Wq=_fake(2), g=_fake(3), b=_fake(4), C=_fake(5), Cp=_fake(6), V=_fake(7), y=_fake(8))
    args.update(over)
    sv = over.get("saved", L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14)))
    ws = over.get("ws", _fake(15))
    ws_bytes = over.get("ws_bytes", 16)
    return L.lib().pkm_forward(h.ptr, None, T, args["x"], args["Wq"], args["g"], args["b"], args["C"], args["Cp"],
                               args["V"], args["y"], ctypes.byref(sv), ws, ws_bytes)


def test_forward_argument_errors():
    L = _lib()
    h = L.pkm_create(_cfg(L))
    assert _fwd(L, h, x=None) == L.PKM_ERR_INVALID_ARG
    assert "x is NULL" in L.lib().pkm_last_error().decode()
    assert _fwd(L, h, V=ctypes.c_void_p(FAKE + 8)) == L.PKM_ERR_INVALID_ARG     # misaligned
    assert "aligned" in L.lib().pkm_last_error().decode()
    assert _fwd(L, h, g=None) == L.PKM_ERR_INVALID_ARG                           # BN needs gamma
    assert _fwd(L, h, T=-5) == L.PKM_ERR_INVALID_ARG
    assert _fwd(L, h, ws=None) == L.PKM_ERR_WORKSPACE
    assert _fwd(L, h, ws_bytes=16) == L.PKM_ERR_WORKSPACE                       # too small
    assert "needed" in L.lib().pkm_last_error().decode()
    bad_saved = L.pkm_saved(_fake(9), None, _fake(11), _fake(12), _fake(13), _fake(14))
    assert _fwd(L, h, saved=bad_saved) == L.PKM_ERR_INVALID_ARG
    assert L.lib().pkm_forward(None, None, 1, *([None] * 8), None, None, 0) == L.PKM_ERR_INVALID_ARG


def test_backward_and_stage_argument_errors():
    L = _lib()
    lib = L.lib()
    h = L.pkm_create(_cfg(L))
    sv = L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14))
    ok = [_fake(i) for i in range(30)]
    # backward: NULL n_touched, then a too-small workspace
    st = lib.pkm_backward(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv), ok[8],
                          ok[9], None, ok[11], ok[12], ok[13], ok[14], ok[15], None, ok[16], 16)
    assert st == L.PKM_ERR_INVALID_ARG
    st = lib.pkm_backward(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv), ok[8],
                          ok[9], ok[10], ok[11], ok[12], ok[13], ok[14], ok[15], None, ok[16], 16)
    assert st == L.PKM_ERR_WORKSPACE
    assert lib.pkm_stage_gather(h.ptr, None, 4, ok[1], None, ok[3], ok[4]) == L.PKM_ERR_INVALID_ARG
    assert lib.pkm_stage_score_topk(h.ptr, None, 4, ok[1], ok[2], None, ok[4], ok[5], ok[6], 1 << 30) == \
        L.PKM_ERR_INVALID_ARG
    assert lib.pkm_stage_merge_softmax(h.ptr, None, 4, ok[1], ok[2], ok[3], ctypes.c_void_p(FAKE + 4),
                                       None) == L.PKM_ERR_INVALID_ARG
    assert lib.pkm_stage_value_grad(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ok[8], ok[9],
                                    16) == L.PKM_ERR_WORKSPACE
    assert lib.pkm_stage_subkey_grad(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ok[8], ok[9],
                                     None, 0) == L.PKM_ERR_WORKSPACE
    assert lib.pkm_stage_query_grad(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ctypes.byref(sv), ok[5], None,
                                    ok[7], None, ok[9], 1 << 30) == L.PKM_ERR_INVALID_ARG   # BN needs dgamma
    assert lib.pkm_stage_query(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ctypes.byref(sv), ok[5],
                               16) == L.PKM_ERR_WORKSPACE
    assert lib.pkm_stage_row_groups(h.ptr, None, 4, ok[1], ok[2], None, ok[3], 1 << 30) == L.PKM_ERR_INVALID_ARG
    assert lib.pkm_stage_row_groups(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], 16) == L.PKM_ERR_WORKSPACE
    assert lib.pkm_stage_value_grad_grouped(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], None, ok[6],
                                            1 << 30) == L.PKM_ERR_INVALID_ARG
    assert lib.pkm_stage_value_grad_grouped(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7],
                                            16) == L.PKM_ERR_WORKSPACE
    for s in range(5):
        assert lib.pkm_status_string(s)


def test_adam_argument_errors():
    L = _lib()
    lib = L.lib()
    h = L.pkm_create(_cfg(L))
    sv = L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14))
    ok = [_fake(i) for i in range(30)]

    def stage(hp, ws_bytes=16):
        ref = ctypes.byref(hp) if hp is not None else None
        return lib.pkm_stage_value_adam(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ref, ok[7], ok[8],
                                        ok[9], ok[10], ws_bytes)

    good = dict(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1)
    assert stage(L.pkm_adam(**good)) == L.PKM_ERR_WORKSPACE       # every other check passes
    assert stage(None) == L.PKM_ERR_INVALID_ARG
    for field, bad in (("lr", float("nan")), ("lr", -1.0), ("beta1", 1.0), ("beta2", -0.1), ("eps", 0.0),
                       ("step", 0)):
        hp = L.pkm_adam(**{**good, field: bad})
        assert stage(hp) == L.PKM_ERR_INVALID_ARG, field
        assert field in lib.pkm_last_error().decode()
    st = lib.pkm_backward_adam(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv),
                               ok[8], ok[9], ctypes.byref(L.pkm_adam(**good)), ok[10], ok[11], ok[12], ok[13],
                               ok[14], ok[15], ok[16], None, ok[17], 16)
    assert st == L.PKM_ERR_WORKSPACE
    grouped = lib.pkm_stage_value_adam_grouped
    assert grouped(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ctypes.byref(L.pkm_adam(**good)), ok[6], ok[7],
                   ok[8], 16) == L.PKM_ERR_WORKSPACE
    assert grouped(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ctypes.byref(L.pkm_adam(**{**good, "step": 0})),
                   ok[6], ok[7], ok[8], 1 << 40) == L.PKM_ERR_INVALID_ARG
    st = lib.pkm_backward_adam(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv),
                               None, ok[9], ctypes.byref(L.pkm_adam(**good)), ok[10], ok[11], ok[12], ok[13],
                               ok[14], ok[15], ok[16], None, ok[17], 1 << 40)
    assert st == L.PKM_ERR_INVALID_ARG and "adam_m" in lib.pkm_last_error().decode()



def test_adam_rows_argument_errors():
    L = _lib()
    lib = L.lib()
    h = L.pkm_create(_cfg(L))
    sv = L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14))
    ok = [_fake(i) for i in range(30)]
    hp = L.pkm_adam(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=1)
    slots = h.cfg.n_keys * h.cfg.n_keys2

    def state(**over):
        f = dict(slot=_fake(20), m=_fake(21), v=_fake(22), n_used=_fake(23), capacity=slots)
        f.update(over)
        return L.pkm_adam_rows(f["slot"], f["m"], f["v"], f["n_used"], f["capacity"])

    def stage(st, adam=hp, ws_bytes=16):
        ref = ctypes.byref(st) if st is not None else None
        return lib.pkm_stage_value_adam_rows(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ref, ctypes.byref(adam),
                                             ok[7], ok[8], ok[9], ok[10], ws_bytes)

    assert stage(state()) == L.PKM_ERR_WORKSPACE                  # every other check passes
    assert stage(state(capacity=0)) == L.PKM_ERR_WORKSPACE        # an empty pool is allowed
    assert stage(state(capacity=0, m=None, v=None)) == L.PKM_ERR_WORKSPACE
    assert stage(None) == L.PKM_ERR_INVALID_ARG
    for field in ("slot", "m", "v", "n_used"):   # m and v are needed for a pool of rows
        assert stage(state(**{field: None})) == L.PKM_ERR_INVALID_ARG, field
        assert f"state.{field}" in lib.pkm_last_error().decode()
    assert stage(state(n_used=ctypes.c_void_p(FAKE + 4))) == L.PKM_ERR_INVALID_ARG
    assert "aligned" in lib.pkm_last_error().decode()
    for cap in (-1, slots + 1):
        assert stage(state(capacity=cap)) == L.PKM_ERR_INVALID_ARG, cap
        assert "capacity" in lib.pkm_last_error().decode()
    assert stage(state(), adam=L.pkm_adam(lr=1e-3, beta1=0.9, beta2=0.999, eps=1e-8, step=0)) == \
        L.PKM_ERR_INVALID_ARG
    bwd = lib.pkm_backward_adam_rows
    st = bwd(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv),
             ctypes.byref(state()), ctypes.byref(hp), ok[10], ok[11], ok[12], ok[13], ok[14], ok[15], ok[16], None,
             ok[17], 16)
    assert st == L.PKM_ERR_WORKSPACE
    st = bwd(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv), None,
             ctypes.byref(hp), ok[10], ok[11], ok[12], ok[13], ok[14], ok[15], ok[16], None, ok[17], 1 << 40)
    assert st == L.PKM_ERR_INVALID_ARG and "state" in lib.pkm_last_error().decode()

def test_diagnostics_argument_errors():
    L = _lib()
    lib = L.lib()
    h = L.pkm_create(_cfg(L))
    ok = [_fake(i) for i in range(12)]
    d = lib.pkm_diagnostics
    assert d(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], None, None, ok[6], 16) == L.PKM_ERR_WORKSPACE
    assert d(h.ptr, None, 4, ok[1], None, ok[3], ok[4], ok[5], None, None, ok[6], 1 << 30) == L.PKM_ERR_INVALID_ARG
    assert d(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], None, None, None, ok[6], 1 << 30) == L.PKM_ERR_INVALID_ARG
    assert "used" in lib.pkm_last_error().decode()
    assert d(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ctypes.c_void_p(FAKE + 4), None, None, ok[6],
             1 << 30) == L.PKM_ERR_INVALID_ARG                                              # misaligned used
    assert d(h.ptr, None, -1, ok[1], ok[2], ok[3], ok[4], ok[5], None, None, ok[6], 1 << 30) == L.PKM_ERR_INVALID_ARG


def test_fp8_values_argument_errors():
    L = _lib()
    lib = L.lib()
    cfg = _cfg(L, values="fp8", d_value=64)
    bad = _cfg(L, values="fp8", d_value=64)
    bad.value_format = 2
    assert lib.pkm_create(ctypes.byref(bad), ctypes.byref(ctypes.c_void_p())) == L.PKM_ERR_INVALID_ARG
    h = L.pkm_create(cfg)
    ok = [_fake(i) for i in range(30)]
    q = lib.pkm_quantize_values
    assert q(h.ptr, None, ok[1], -1, ok[2]) == L.PKM_ERR_INVALID_ARG
    assert q(h.ptr, None, ok[1], 32 * 32 + 1, ok[2]) == L.PKM_ERR_INVALID_ARG      # more rows than the table
    assert q(h.ptr, None, None, 4, ok[2]) == L.PKM_ERR_INVALID_ARG
    assert q(h.ptr, None, ok[1], 0, ok[2]) == L.PKM_OK                              # nothing to do
    plain = L.pkm_create(_cfg(L))
    assert q(plain.ptr, None, ok[1], 4, ok[2]) == L.PKM_ERR_INVALID_ARG           # needs an fp8 handle
    # every entry point that reads V in the backward refuses fp8 values
    sv = L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14))
    st = lib.pkm_backward(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv), ok[8],
                          ok[9], ok[10], ok[11], ok[12], ok[13], ok[14], ok[15], None, ok[16], 1 << 40)
    assert st == L.PKM_ERR_UNSUPPORTED and "fp8" in lib.pkm_last_error().decode()
    assert lib.pkm_stage_value_grad(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ok[8], ok[9],
                                    1 << 40) == L.PKM_ERR_UNSUPPORTED
    assert lib.pkm_stage_value_grad_grouped(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7],
                                            1 << 40) == L.PKM_ERR_UNSUPPORTED


def test_idw_scores_and_fwpkm_chunk_argument_errors():
    L = _lib()
    lib = L.lib()
    bad = _cfg(L, score="idw")
    bad.score_fn = 3
    assert lib.pkm_create(ctypes.byref(bad), ctypes.byref(ctypes.c_void_p())) == L.PKM_ERR_INVALID_ARG
    h = L.pkm_create(_cfg(L, score="idw"))
    dot = L.pkm_create(_cfg(L))
    assert L.pkm_get_config(h).score_fn == L.PKM_SCORE_IDW
    # the chunk's workspace holds the forward's and the backward's, plus the residual and the touched rows
    T = 500
    fwd, bwd = L.pkm_workspace_size(h, T, L.PKM_WS_FORWARD), L.pkm_workspace_size(h, T, L.PKM_WS_BACKWARD)
    chunk = L.pkm_workspace_size(h, T, L.PKM_WS_FWPKM_CHUNK)
    assert chunk >= max(fwd, bwd) + T * 64 * 4 + T * 2 * 8 * 4
    with pytest.raises(L.PkmError) as e:
        L.pkm_workspace_size(h, T, 3)
    assert e.value.status == L.PKM_ERR_INVALID_ARG
    ok = [_fake(i) for i in range(30)]
    big = 1 << 40
    c = lib.pkm_fwpkm_chunk

    def call(handle=h, T=10, lr=0.1, ws_bytes=big, streams=1, **over):
        a = [over.get(n, ok[i]) for i, n in enumerate(("q", "C", "Cp", "V", "target", "y", "idx", "w"), 1)]
        return c(handle.ptr, None, T, streams, a[0], a[1], a[2], a[3], a[4], lr, a[5], a[6], a[7], ok[20], ws_bytes)

    assert call(handle=dot) == L.PKM_ERR_UNSUPPORTED and "IDW" in lib.pkm_last_error().decode()
    for n in ("q", "C", "Cp", "V", "target", "y", "idx", "w"):
        assert call(**{n: None}) == L.PKM_ERR_INVALID_ARG, n
        assert n in lib.pkm_last_error().decode()
    assert call(q=ctypes.c_void_p(FAKE + 4)) == L.PKM_ERR_INVALID_ARG              # misaligned
    for lr in (-0.5, float("inf"), float("nan")):
        assert call(lr=lr) == L.PKM_ERR_INVALID_ARG
    assert call(ws_bytes=16) == L.PKM_ERR_WORKSPACE
    assert call(T=-1) == L.PKM_ERR_INVALID_ARG
    assert call(T=0) == L.PKM_OK                                                     # nothing to do
    # a batch of streams: T a multiple of streams, every stream's rows addressable as int32
    assert call(streams=0) == L.PKM_ERR_INVALID_ARG
    assert call(T=10, streams=3) == L.PKM_ERR_INVALID_ARG
    assert "multiple" in lib.pkm_last_error().decode()
    assert call(T=12, streams=3, ws_bytes=16) == L.PKM_ERR_WORKSPACE                 # the other checks pass
    big_keys = L.pkm_create(_cfg(L, score="idw", n_keys=2048, n_keys2=2048))
    assert call(handle=big_keys, T=1024, streams=512) == L.PKM_ERR_UNSUPPORTED       # 512 * 2^22 = 2^31 rows
    assert call(handle=big_keys, T=1022, streams=511, ws_bytes=16) == L.PKM_ERR_WORKSPACE  # fits: next check
    fp8 = L.pkm_create(_cfg(L, score="idw", values="fp8", d_value=64))
    assert call(handle=fp8) == L.PKM_ERR_UNSUPPORTED
    # several calls in one: T a multiple of call_T, call_T a multiple of streams
    cs = lib.pkm_fwpkm_chunks

    def calls(T=12, call_T=6, streams=1, ws_bytes=big, handle=h):
        return cs(handle.ptr, None, T, call_T, streams, *ok[1:6], 0.1, *ok[6:9], ok[20], ws_bytes)

    assert calls(call_T=0) == L.PKM_ERR_INVALID_ARG
    assert calls(call_T=5) == L.PKM_ERR_INVALID_ARG and "multiple" in lib.pkm_last_error().decode()
    assert calls(call_T=6, streams=4) == L.PKM_ERR_INVALID_ARG and "multiple" in lib.pkm_last_error().decode()
    assert calls(handle=dot) == L.PKM_ERR_UNSUPPORTED
    assert calls(T=0) == L.PKM_OK
    assert calls(call_T=6, streams=3, ws_bytes=16) == L.PKM_ERR_WORKSPACE           # the other checks pass
    assert calls(ws_bytes=L.pkm_workspace_size(h, 6, L.PKM_WS_FWPKM_CHUNK)) == L.PKM_ERR_WORKSPACE  # sized for T
    # the score gradients are the dot product's: the backward refuses IDW handles
    sv = L.pkm_saved(_fake(9), _fake(10), _fake(11), _fake(12), _fake(13), _fake(14))
    st = lib.pkm_backward(h.ptr, None, 10, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ctypes.byref(sv), ok[8],
                          ok[9], ok[10], ok[11], ok[12], ok[13], ok[14], ok[15], None, ok[16], big)
    assert st == L.PKM_ERR_UNSUPPORTED and "dot-product" in lib.pkm_last_error().decode()
    assert lib.pkm_stage_subkey_grad(h.ptr, None, 4, ok[1], ok[2], ok[3], ok[4], ok[5], ok[6], ok[7], ok[8], ok[9],
                                     ok[10], big) == L.PKM_ERR_UNSUPPORTED


def test_binding_rejects_host_tensors():
    L = _lib()
    import torch
    h = L.pkm_create(_cfg(L))
    with pytest.raises(ValueError):
        L.pkm_stage_gather(h, 1, torch.zeros(8, dtype=torch.int32), torch.zeros(8), torch.zeros(64),
                           torch.zeros(64))


def _t(n, dtype=None):
    import torch
    return torch.zeros(max(0, n), dtype=dtype if dtype is not None else torch.float32)


def test_binding_rejects_short_tensors_before_the_library():
    # every size check runs before the device check: a short host tensor names itself, a full-size set of
    # host tensors gets as far as "must be on the GPU"
    L = _lib()
    import torch
    c = _cfg(L)
    h = L.pkm_create(c)
    T = 10
    F, half, slots = c.heads * c.d_query, c.d_query // 2, c.n_keys * c.n_keys2
    lk = T * c.heads * c.topk
    i32 = torch.int32

    def fwd(**over):
        a = dict(x=_t(T * c.d_in), Wq=_t(F * c.d_in), g=_t(F), b=_t(F), C=_t(c.heads * c.n_keys * half),
                 Cp=_t(c.heads * c.n_keys2 * half), V=_t(slots * c.d_value), y=_t(T * c.d_value))
        a.update(over)
        saved = {"idx": _t(lk, i32), "w": _t(lk), "q": _t(T * F), "q_pre": _t(T * F), "bn_mean": _t(F),
                 "bn_rstd": _t(F)}
        saved.update(a.pop("saved", {}))
        L.pkm_forward(h, T, a["x"], a["Wq"], a["g"], a["b"], a["C"], a["Cp"], a["V"], a["y"], saved, None)

    with pytest.raises(ValueError, match="on the GPU"):
        fwd()
    for name, short in (("x", _t(T * c.d_in - 1)), ("V", _t(slots * c.d_value - 4)), ("y", _t(c.d_value)),
                        ("Cp", _t(3)), ("g", _t(F - 1))):
        with pytest.raises(ValueError, match="holds"):
            fwd(**{name: short})
    with pytest.raises(ValueError, match="holds"):
        fwd(saved={"idx": _t(lk - 1, i32)})

    # the value gradient stage: V and dV cover every slot, idx/w/dw every lookup
    def vg(**over):
        a = dict(idx=_t(lk, i32), w=_t(lk), dY=_t(T * c.d_value), V=_t(slots * c.d_value),
                 dV=_t(slots * c.d_value), touched=_t(lk, i32), nt=_t(1, torch.int64), dw=_t(lk))
        a.update(over)
        L.pkm_stage_value_grad(h, T, a["idx"], a["w"], a["dY"], a["V"], a["dV"], a["touched"], a["nt"], a["dw"], None)

    with pytest.raises(ValueError, match="on the GPU"):
        vg()
    for name in ("idx", "w", "dY", "V", "dV", "touched", "dw"):
        with pytest.raises(ValueError, match="holds"):
            vg(**{name: _t(5, i32 if name in ("idx", "touched") else None)})

    # the memorization chunk: V holds streams * |C| * |C'| rows
    hi = L.pkm_create(_cfg(L, score="idw", bn=False))

    def chunk(streams, **over):
        a = dict(q=_t(T * F), C=_t(c.heads * c.n_keys * half), Cp=_t(c.heads * c.n_keys2 * half),
                 V=_t(streams * slots * c.d_value), target=_t(T * c.d_value), y=_t(T * c.d_value), idx=_t(lk, i32),
                 w=_t(lk))
        a.update(over)
        L.pkm_fwpkm_chunk(hi, T, a["q"], a["C"], a["Cp"], a["V"], a["target"], 0.1, a["y"], a["idx"], a["w"], None,
                          streams=streams)

    with pytest.raises(ValueError, match="on the GPU"):
        chunk(2)
    with pytest.raises(ValueError, match="holds"):
        chunk(2, V=_t(slots * c.d_value))
    with pytest.raises(ValueError, match="holds"):
        chunk(1, target=_t(T * c.d_value - 1))
    with pytest.raises(ValueError):
        chunk(0)


def test_forward_noalloc_rejects_oversize_T_before_any_device_call():
    # the workspace check precedes the pointer checks and the scratch lookup
    L = _lib()
    lib = L.lib()
    h = L.pkm_create(_cfg(L, d_in=64, heads=4, d_query=512, n_keys=1024, n_keys2=1024, topk=32, d_value=64,
                          dtype="bf16"))
    T = 60000
    assert L.pkm_workspace_size(h, T, 0) > 128 << 20
    st = lib.pkm_forward_noalloc(h.ptr, None, T, None, None, None, None, None, None, None, None, None)
    assert st == L.PKM_ERR_WORKSPACE and "scratch" in lib.pkm_last_error().decode()
    # within the limit, the NULL pointers are what it rejects
    assert lib.pkm_forward_noalloc(h.ptr, None, 1000, None, None, None, None, None, None, None, None,
                                   None) == L.PKM_ERR_INVALID_ARG
