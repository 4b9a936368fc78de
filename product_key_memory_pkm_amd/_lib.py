"""ctypes binding of libpkm.so (the C ABI in include/pkm.h).

Argument marshalling only: every function here checks that torch tensors sit
on the GPU with the expected dtype and layout, turns them into raw pointers and
calls the C entry point of the same name on torch's current stream.  All
arithmetic happens in the library's HIP kernels; there is no fallback.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
# PKM_LIB_PATH names another build of the same library (the CPU tests load a
# copy whose host code carries address and undefined-behaviour checks)
LIB_PATH = os.environ.get("PKM_LIB_PATH") or os.path.join(_HERE, "libpkm.so")

PKM_OK, PKM_ERR_INVALID_ARG, PKM_ERR_UNSUPPORTED, PKM_ERR_WORKSPACE, PKM_ERR_HIP = range(5)
PKM_F32, PKM_BF16 = 0, 1
PKM_BN_NONE, PKM_BN_BATCH = 0, 1
PKM_VALUES_STORAGE, PKM_VALUES_FP8 = 0, 1
PKM_SCORE_DOT, PKM_SCORE_IDW = 0, 1
PKM_WS_FORWARD, PKM_WS_BACKWARD, PKM_WS_FWPKM_CHUNK = 0, 1, 2

_STORAGE = {PKM_F32: torch.float32, PKM_BF16: torch.bfloat16}


class PkmError(RuntimeError):
    def __init__(self, status: int, func: str, msg: str):
        super().__init__(f"{func}: status {status} ({msg})")
        self.status = status


class pkm_config(ctypes.Structure):
    _fields_ = [("d_in", ctypes.c_int32), ("heads", ctypes.c_int32), ("d_query", ctypes.c_int32),
                ("n_keys", ctypes.c_int32), ("n_keys2", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("d_value", ctypes.c_int32), ("dtype", ctypes.c_int32), ("bn", ctypes.c_int32),
                ("bn_eps", ctypes.c_float), ("temperature", ctypes.c_float), ("accumulate_dv", ctypes.c_int32),
                ("value_format", ctypes.c_int32), ("score_fn", ctypes.c_int32)]


class pkm_saved(ctypes.Structure):
    _fields_ = [("idx", ctypes.c_void_p), ("w", ctypes.c_void_p), ("q", ctypes.c_void_p),
                ("q_pre", ctypes.c_void_p), ("bn_mean", ctypes.c_void_p), ("bn_rstd", ctypes.c_void_p)]


class pkm_adam(ctypes.Structure):
    _fields_ = [("lr", ctypes.c_float), ("beta1", ctypes.c_float), ("beta2", ctypes.c_float),
                ("eps", ctypes.c_float), ("step", ctypes.c_int64)]


class pkm_adam_rows(ctypes.Structure):
    _fields_ = [("slot", ctypes.c_void_p), ("m", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("n_used", ctypes.c_void_p), ("capacity", ctypes.c_int64)]


_lib = None

# name -> argument types (all return pkm_status as int)
_VP, _I64, _SZ = ctypes.c_void_p, ctypes.c_int64, ctypes.c_size_t
_SIGS = {
    "pkm_create": [ctypes.POINTER(pkm_config), ctypes.POINTER(ctypes.c_void_p)],
    "pkm_destroy": [_VP],
    "pkm_get_config": [_VP, ctypes.POINTER(pkm_config)],
    "pkm_workspace_size": [_VP, _I64, ctypes.c_int, ctypes.POINTER(ctypes.c_size_t)],
    "pkm_forward": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved), _VP, _SZ],
    "pkm_forward_noalloc": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved)],
    "pkm_backward": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved), _VP, _VP, _VP,
                     _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_backward_adam": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved), _VP, _VP,
                          ctypes.POINTER(pkm_adam), _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_backward_adam_rows": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved),
                               ctypes.POINTER(pkm_adam_rows), ctypes.POINTER(pkm_adam), _VP, _VP, _VP, _VP, _VP, _VP,
                               _VP, _VP, _VP, _SZ],
    "pkm_stage_query": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved), _VP, _SZ],
    "pkm_stage_score_topk": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_stage_merge_softmax": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP],
    "pkm_stage_gather": [_VP, _VP, _I64, _VP, _VP, _VP, _VP],
    "pkm_stage_value_grad": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_stage_value_adam": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_adam), _VP, _VP, _VP,
                             _VP, _SZ],
    "pkm_stage_value_adam_grouped": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_adam), _VP, _VP,
                                     _VP, _SZ],
    "pkm_stage_value_adam_rows": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_adam_rows),
                                  ctypes.POINTER(pkm_adam), _VP, _VP, _VP, _VP, _SZ],
    "pkm_diagnostics": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_quantize_values": [_VP, _VP, _VP, _I64, _VP],
    "pkm_stage_row_groups": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _SZ],
    "pkm_stage_value_grad_grouped": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_stage_subkey_grad": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _VP, _SZ],
    "pkm_stage_query_grad": [_VP, _VP, _I64, _VP, _VP, _VP, _VP, ctypes.POINTER(pkm_saved), _VP, _VP, _VP, _VP,
                             _VP, _SZ],
    "pkm_fwpkm_chunk": [_VP, _VP, _I64, _I64, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP, _VP, _SZ],
    "pkm_fwpkm_chunks": [_VP, _VP, _I64, _I64, _I64, _VP, _VP, _VP, _VP, _VP, ctypes.c_float, _VP, _VP, _VP, _VP,
                         _SZ],
}
EXPORTED = sorted(list(_SIGS) + ["pkm_status_string", "pkm_last_error"])


def lib() -> ctypes.CDLL:
    """Load libpkm.so (built in place by ``product_key_memory_pkm_amd.build``); fail loudly if absent."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -m product_key_memory_pkm_amd.build`")
        L = ctypes.CDLL(LIB_PATH)
        for name, args in _SIGS.items():
            f = getattr(L, name)
            f.argtypes = args
            f.restype = ctypes.c_int
        L.pkm_status_string.argtypes = [ctypes.c_int]
        L.pkm_status_string.restype = ctypes.c_char_p
        L.pkm_last_error.argtypes = []
        L.pkm_last_error.restype = ctypes.c_char_p
        _lib = L
    return _lib


def _check(status: int, func: str) -> None:
    if status != PKM_OK:
        L = lib()
        raise PkmError(status, func, L.pkm_last_error().decode() or L.pkm_status_string(status).decode())


def _ptr(t):
    if t is None:
        return None
    if not isinstance(t, torch.Tensor):
        raise TypeError("expected a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError("tensor must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensor must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device=None) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def _invoke(name: str, h, T: int, *args) -> int:
    """Call ``name(handle, stream, T, *args)`` on torch's current stream (arguments already marshalled)."""
    return getattr(lib(), name)(h.ptr, _stream(), T, *args)


def _dt(t, want, name):
    if t is not None and t.dtype != want:
        raise TypeError(f"{name} must be {want}, got {t.dtype}")


def _need(**req):
    """Each keyword is (tensor or None, elements the call reads or writes): a shorter tensor raises ValueError
    before anything reaches the library, whose kernels trust the sizes pkm.h states."""
    for name, (t, n) in req.items():
        if t is not None and t.numel() < n:
            raise ValueError(f"{name} holds {t.numel()} elements; this call needs {n}")


def fp8_row_bytes(d_value: int) -> int:
    """Bytes of one fp8 value row (pkm.h PKM_FP8_ROW_BYTES): d_value + 16 rounded up to a multiple of 128."""
    return (d_value + 16 + 127) // 128 * 128


def _dims(h, T: int, streams: int = 1) -> dict:
    """Element counts of the buffers pkm.h describes, for handle ``h`` and T tokens."""
    c = h.cfg
    F = c.heads * c.d_query
    half = c.d_query // 2
    slots = c.n_keys * c.n_keys2 * streams
    vrow = fp8_row_bytes(c.d_value) if c.value_format == PKM_VALUES_FP8 else c.d_value
    return {"x": T * c.d_in, "Wq": F * c.d_in, "F": F, "C": c.heads * c.n_keys * half,
            "Cp": c.heads * c.n_keys2 * half, "V": slots * vrow, "dV": slots * c.d_value, "y": T * c.d_value,
            "lookups": T * c.heads * c.topk, "sub": T * c.heads * 2 * c.topk, "q": T * F,
            "hits_c": c.heads * c.n_keys, "hits_cp": c.heads * c.n_keys2, "used": 1 + c.heads,
            "th": T * c.heads}


def _need_saved(h, T: int, saved: dict):
    """The saved state: idx, w [T, h, k]; q, q_pre [T, h*dq]; bn_mean, bn_rstd [h*dq] (BatchNorm only)."""
    n = _dims(h, T)
    req = {"saved['idx']": (saved.get("idx"), n["lookups"]), "saved['w']": (saved.get("w"), n["lookups"]),
           "saved['q']": (saved.get("q"), n["q"]), "saved['q_pre']": (saved.get("q_pre"), n["q"])}
    if h.cfg.bn == PKM_BN_BATCH:
        req.update({"saved['bn_mean']": (saved.get("bn_mean"), n["F"]),
                    "saved['bn_rstd']": (saved.get("bn_rstd"), n["F"])})
    _need(**req)


class Handle:
    """An immutable PKM layer handle (host memory only)."""

    def __init__(self, ptr: int, cfg: pkm_config):
        self.ptr = ctypes.c_void_p(ptr)
        self.cfg = cfg

    @property
    def storage(self) -> torch.dtype:
        return _STORAGE[self.cfg.dtype]

    @property
    def value_dtype(self) -> torch.dtype:
        """dtype of the value table tensor: the storage dtype, or uint8 bytes for fp8 rows."""
        return torch.uint8 if self.cfg.value_format == PKM_VALUES_FP8 else self.storage

    def __del__(self):
        if _lib is not None and self.ptr:
            _lib.pkm_destroy(self.ptr)
            self.ptr = ctypes.c_void_p(None)


def make_config(d_in, heads, d_query, n_keys, n_keys2, topk, d_value, dtype="f32", bn=True, bn_eps=1e-5,
                temperature=1.0, accumulate_dv=True, values="storage", score="dot") -> pkm_config:
    """``values``: "storage" (V in the storage dtype) or "fp8" (rows of a fp32 scale + E4M3 codes);
    ``score``: "dot" (q . c) or "idw" (-log ||q - c||, the fast-weight memory's scores)."""
    if values not in ("storage", "fp8"):
        raise ValueError(f"values must be 'storage' or 'fp8', got {values!r}")
    if score not in ("dot", "idw"):
        raise ValueError(f"score must be 'dot' or 'idw', got {score!r}")
    return pkm_config(d_in, heads, d_query, n_keys, n_keys2, topk, d_value,
                      PKM_BF16 if dtype in ("bf16", PKM_BF16, torch.bfloat16) else PKM_F32,
                      PKM_BN_BATCH if bn else PKM_BN_NONE, bn_eps, temperature, 1 if accumulate_dv else 0,
                      PKM_VALUES_FP8 if values == "fp8" else PKM_VALUES_STORAGE,
                      PKM_SCORE_IDW if score == "idw" else PKM_SCORE_DOT)


def pkm_create(cfg: pkm_config) -> Handle:
    out = ctypes.c_void_p()
    _check(lib().pkm_create(ctypes.byref(cfg), ctypes.byref(out)), "pkm_create")
    return Handle(out.value, cfg)


def pkm_get_config(h: Handle) -> pkm_config:
    c = pkm_config()
    _check(lib().pkm_get_config(h.ptr, ctypes.byref(c)), "pkm_get_config")
    return c


def pkm_workspace_size(h: Handle, T: int, with_backward) -> int:
    """``with_backward``: False/True (forward / backward) or one of PKM_WS_FORWARD, PKM_WS_BACKWARD,
    PKM_WS_FWPKM_CHUNK."""
    kind = int(with_backward)
    n = ctypes.c_size_t()
    _check(lib().pkm_workspace_size(h.ptr, T, kind, ctypes.byref(n)), "pkm_workspace_size")
    return n.value


def _saved_struct(saved: dict) -> pkm_saved:
    return pkm_saved(*[_ptr(saved.get(k)) for k in ("idx", "w", "q", "q_pre", "bn_mean", "bn_rstd")])


def _nbytes(t):
    return 0 if t is None else t.numel() * t.element_size()


def pkm_forward(h, T, x, Wq, bn_gamma, bn_beta, C, Cp, V, y, saved: dict, ws):
    st = h.storage
    for n, t in (("x", x), ("Wq", Wq), ("C", C), ("Cp", Cp), ("y", y)):
        _dt(t, st, n)
    _dt(V, h.value_dtype, "V")
    n = _dims(h, T)
    _need(x=(x, n["x"]), Wq=(Wq, n["Wq"]), bn_gamma=(bn_gamma, n["F"]), bn_beta=(bn_beta, n["F"]), C=(C, n["C"]),
          Cp=(Cp, n["Cp"]), V=(V, n["V"]), y=(y, n["y"]))
    _need_saved(h, T, saved)
    sv = _saved_struct(saved)
    _check(_invoke("pkm_forward", h, T, _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(bn_beta), _ptr(C),
                             _ptr(Cp), _ptr(V), _ptr(y), ctypes.byref(sv), _ptr(ws), _nbytes(ws)), "pkm_forward")


def pkm_forward_noalloc(h, T, x, Wq, bn_gamma, bn_beta, C, Cp, V, y, saved: dict):
    """pkm_forward with the library's static per-device scratch as its workspace (pkm.h): for callers that
    cannot allocate.  Calls that overlap in time on one GPU race on that scratch."""
    st = h.storage
    for n, t in (("x", x), ("Wq", Wq), ("C", C), ("Cp", Cp), ("y", y)):
        _dt(t, st, n)
    _dt(V, h.value_dtype, "V")
    n = _dims(h, T)
    _need(x=(x, n["x"]), Wq=(Wq, n["Wq"]), bn_gamma=(bn_gamma, n["F"]), bn_beta=(bn_beta, n["F"]), C=(C, n["C"]),
          Cp=(Cp, n["Cp"]), V=(V, n["V"]), y=(y, n["y"]))
    _need_saved(h, T, saved)
    sv = _saved_struct(saved)
    _check(_invoke("pkm_forward_noalloc", h, T, _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(bn_beta), _ptr(C), _ptr(Cp),
                   _ptr(V), _ptr(y), ctypes.byref(sv)), "pkm_forward_noalloc")


def pkm_backward(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved: dict, dV, touched, n_touched, dC, dCp, dWq, dgamma,
                 dbeta, dx, ws):
    st = h.storage
    for n, t in (("dY", dY), ("x", x), ("Wq", Wq), ("C", C), ("Cp", Cp), ("V", V), ("dx", dx)):
        _dt(t, st, n)
    _dt(dV, torch.float32, "dV")
    _dt(n_touched, torch.int64, "n_touched")
    _need_bwd(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, touched, n_touched, dC, dCp, dWq, dgamma, dbeta, dx)
    _need(dV=(dV, _dims(h, T)["dV"]))
    sv = _saved_struct(saved)
    _check(_invoke("pkm_backward", h, T, _ptr(dY), _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(C), _ptr(Cp),
                              _ptr(V), ctypes.byref(sv), _ptr(dV), _ptr(touched), _ptr(n_touched), _ptr(dC),
                              _ptr(dCp), _ptr(dWq), _ptr(dgamma), _ptr(dbeta), _ptr(dx), _ptr(ws), _nbytes(ws)),
           "pkm_backward")


def _need_bwd(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, touched, n_touched, dC, dCp, dWq, dgamma, dbeta, dx):
    n = _dims(h, T)
    _need(dY=(dY, n["y"]), x=(x, n["x"]), Wq=(Wq, n["Wq"]), bn_gamma=(bn_gamma, n["F"]), C=(C, n["C"]),
          Cp=(Cp, n["Cp"]), V=(V, n["V"]), touched=(touched, n["lookups"]), n_touched=(n_touched, 1),
          dC=(dC, n["C"]), dCp=(dCp, n["Cp"]), dWq=(dWq, n["Wq"]), dgamma=(dgamma, n["F"]),
          dbeta=(dbeta, n["F"]), dx=(dx, n["x"]))
    _need_saved(h, T, saved)


def _adam_struct(adam: dict) -> pkm_adam:
    return pkm_adam(float(adam["lr"]), float(adam["beta1"]), float(adam["beta2"]), float(adam["eps"]),
                    int(adam["step"]))


def pkm_backward_adam(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved: dict, adam_m, adam_v, adam: dict, touched,
                      n_touched, dC, dCp, dWq, dgamma, dbeta, dx, ws):
    """pkm_backward with the Adam step of the touched value rows in place of dV.

    ``adam``: {"lr", "beta1", "beta2", "eps", "step"}; V, adam_m, adam_v are updated in place."""
    st = h.storage
    for n, t in (("dY", dY), ("x", x), ("Wq", Wq), ("C", C), ("Cp", Cp), ("V", V), ("dx", dx)):
        _dt(t, st, n)
    _dt(adam_m, torch.float32, "adam_m")
    _dt(adam_v, torch.float32, "adam_v")
    _dt(n_touched, torch.int64, "n_touched")
    _need_bwd(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, touched, n_touched, dC, dCp, dWq, dgamma, dbeta, dx)
    _need(adam_m=(adam_m, _dims(h, T)["dV"]), adam_v=(adam_v, _dims(h, T)["dV"]))
    sv = _saved_struct(saved)
    hp = _adam_struct(adam)
    _check(_invoke("pkm_backward_adam", h, T, _ptr(dY), _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(C), _ptr(Cp),
                   _ptr(V), ctypes.byref(sv), _ptr(adam_m), _ptr(adam_v), ctypes.byref(hp), _ptr(touched),
                   _ptr(n_touched), _ptr(dC), _ptr(dCp), _ptr(dWq), _ptr(dgamma), _ptr(dbeta), _ptr(dx), _ptr(ws),
                   _nbytes(ws)), "pkm_backward_adam")


def pkm_stage_value_adam(h, T, idx, w, dY, V, adam_m, adam_v, adam: dict, touched, n_touched, dw, ws):
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _dt(adam_m, torch.float32, "adam_m")
    _dt(adam_v, torch.float32, "adam_v")
    _dt(dw, torch.float32, "dw")
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), dY=(dY, n["y"]), V=(V, n["dV"]), adam_m=(adam_m, n["dV"]),
          adam_v=(adam_v, n["dV"]), touched=(touched, n["lookups"]), n_touched=(n_touched, 1),
          dw=(dw, n["lookups"]))
    hp = _adam_struct(adam)
    _check(_invoke("pkm_stage_value_adam", h, T, _ptr(idx), _ptr(w), _ptr(dY), _ptr(V), _ptr(adam_m), _ptr(adam_v),
                   ctypes.byref(hp), _ptr(touched), _ptr(n_touched), _ptr(dw), _ptr(ws), _nbytes(ws)),
           "pkm_stage_value_adam")


def _adam_rows_struct(h, state: dict) -> pkm_adam_rows:
    """state: {"slot": int32 [n_keys * n_keys2], "m", "v": fp32 [capacity, d_value], "n_used": int64 [1]};
    the capacity is the row count of m."""
    c = h.cfg
    _dt(state["slot"], torch.int32, "state['slot']")
    _dt(state["m"], torch.float32, "state['m']")
    _dt(state["v"], torch.float32, "state['v']")
    _dt(state["n_used"], torch.int64, "state['n_used']")
    cap = state["m"].numel() // c.d_value
    _need(**{"state['slot']": (state["slot"], c.n_keys * c.n_keys2), "state['v']": (state["v"], cap * c.d_value),
             "state['n_used']": (state["n_used"], 1)})
    return pkm_adam_rows(_ptr(state["slot"]), _ptr(state["m"]), _ptr(state["v"]), _ptr(state["n_used"]), cap)


def pkm_backward_adam_rows(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved: dict, state: dict, adam: dict, touched,
                           n_touched, dC, dCp, dWq, dgamma, dbeta, dx, ws):
    """pkm_backward_adam with the moments in a pool of slots (``state``, see _adam_rows_struct)."""
    st = h.storage
    for n, t in (("dY", dY), ("x", x), ("Wq", Wq), ("C", C), ("Cp", Cp), ("V", V), ("dx", dx)):
        _dt(t, st, n)
    _dt(n_touched, torch.int64, "n_touched")
    _need_bwd(h, T, dY, x, Wq, bn_gamma, C, Cp, V, saved, touched, n_touched, dC, dCp, dWq, dgamma, dbeta, dx)
    sv = _saved_struct(saved)
    rs = _adam_rows_struct(h, state)
    hp = _adam_struct(adam)
    _check(_invoke("pkm_backward_adam_rows", h, T, _ptr(dY), _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(C), _ptr(Cp),
                   _ptr(V), ctypes.byref(sv), ctypes.byref(rs), ctypes.byref(hp), _ptr(touched), _ptr(n_touched),
                   _ptr(dC), _ptr(dCp), _ptr(dWq), _ptr(dgamma), _ptr(dbeta), _ptr(dx), _ptr(ws), _nbytes(ws)),
           "pkm_backward_adam_rows")


def pkm_stage_value_adam_rows(h, T, idx, w, dY, V, state: dict, adam: dict, touched, n_touched, dw, ws):
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _dt(dw, torch.float32, "dw")
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), dY=(dY, n["y"]), V=(V, n["dV"]),
          touched=(touched, n["lookups"]), n_touched=(n_touched, 1), dw=(dw, n["lookups"]))
    rs = _adam_rows_struct(h, state)
    hp = _adam_struct(adam)
    _check(_invoke("pkm_stage_value_adam_rows", h, T, _ptr(idx), _ptr(w), _ptr(dY), _ptr(V), ctypes.byref(rs),
                   ctypes.byref(hp), _ptr(touched), _ptr(n_touched), _ptr(dw), _ptr(ws), _nbytes(ws)),
           "pkm_stage_value_adam_rows")


def pkm_stage_query(h, T, x, Wq, bn_gamma, bn_beta, saved: dict, ws):
    n = _dims(h, T)
    _need(x=(x, n["x"]), Wq=(Wq, n["Wq"]), bn_gamma=(bn_gamma, n["F"]), bn_beta=(bn_beta, n["F"]),
          **{"saved['q']": (saved.get("q"), n["q"]), "saved['q_pre']": (saved.get("q_pre"), n["q"])},
          **({"saved['bn_mean']": (saved.get("bn_mean"), n["F"]), "saved['bn_rstd']": (saved.get("bn_rstd"), n["F"])}
             if h.cfg.bn == PKM_BN_BATCH else {}))
    sv = _saved_struct(saved)
    _check(_invoke("pkm_stage_query", h, T, _ptr(x), _ptr(Wq), _ptr(bn_gamma), _ptr(bn_beta),
                                 ctypes.byref(sv), _ptr(ws), _nbytes(ws)), "pkm_stage_query")


def pkm_stage_score_topk(h, T, q, C, Cp, sub_idx, sub_score, ws):
    _dt(sub_idx, torch.int32, "sub_idx")
    _dt(sub_score, torch.float32, "sub_score")
    n = _dims(h, T)
    _need(q=(q, n["q"]), C=(C, n["C"]), Cp=(Cp, n["Cp"]), sub_idx=(sub_idx, n["sub"]), sub_score=(sub_score, n["sub"]))
    _check(_invoke("pkm_stage_score_topk", h, T, _ptr(q), _ptr(C), _ptr(Cp), _ptr(sub_idx),
                   _ptr(sub_score), _ptr(ws), _nbytes(ws)), "pkm_stage_score_topk")


def pkm_stage_merge_softmax(h, T, sub_idx, sub_score, idx, w, score=None):
    n = _dims(h, T)
    _need(sub_idx=(sub_idx, n["sub"]), sub_score=(sub_score, n["sub"]), idx=(idx, n["lookups"]), w=(w, n["lookups"]),
          score=(score, n["lookups"]))
    _check(_invoke("pkm_stage_merge_softmax", h, T, _ptr(sub_idx), _ptr(sub_score), _ptr(idx), _ptr(w),
                                         _ptr(score)), "pkm_stage_merge_softmax")


def pkm_quantize_values(h, V_src, V_fp8, rows=None):
    """fp8 rows (fp32 scale + E4M3 codes, padded to fp8_row_bytes(d_value), pkm.h) of the value table
    V_src [rows, d_value] into V_fp8 (uint8)."""
    _dt(V_src, h.storage, "V_src")
    _dt(V_fp8, torch.uint8, "V_fp8")
    n = V_src.shape[0] if rows is None else rows
    if V_fp8.numel() < n * fp8_row_bytes(h.cfg.d_value):
        raise ValueError("V_fp8 holds fewer than rows * PKM_FP8_ROW_BYTES(d_value) bytes")
    _check(lib().pkm_quantize_values(h.ptr, _stream(), _ptr(V_src), n, _ptr(V_fp8)), "pkm_quantize_values")


def pkm_stage_gather(h, T, idx, w, V, y):
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _dt(V, h.value_dtype, "V")
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), V=(V, n["V"]), y=(y, n["y"]))
    _check(_invoke("pkm_stage_gather", h, T, _ptr(idx), _ptr(w), _ptr(V), _ptr(y)), "pkm_stage_gather")


def pkm_stage_value_grad(h, T, idx, w, dY, V, dV, touched, n_touched, dw, ws):
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), dY=(dY, n["y"]), V=(V, n["dV"]), dV=(dV, n["dV"]),
          touched=(touched, n["lookups"]), n_touched=(n_touched, 1), dw=(dw, n["lookups"]))
    _check(_invoke("pkm_stage_value_grad", h, T, _ptr(idx), _ptr(w), _ptr(dY), _ptr(V), _ptr(dV),
                                      _ptr(touched), _ptr(n_touched), _ptr(dw), _ptr(ws), _nbytes(ws)),
           "pkm_stage_value_grad")


def pkm_stage_row_groups(h, T, idx, touched, n_touched, ws):
    _dt(idx, torch.int32, "idx")
    _dt(n_touched, torch.int64, "n_touched")
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), touched=(touched, n["lookups"]), n_touched=(n_touched, 1))
    _check(_invoke("pkm_stage_row_groups", h, T, _ptr(idx), _ptr(touched), _ptr(n_touched), _ptr(ws), _nbytes(ws)),
           "pkm_stage_row_groups")


def pkm_stage_value_grad_grouped(h, T, w, dY, V, dV, dw, n_touched, ws):
    n = _dims(h, T)
    _need(w=(w, n["lookups"]), dY=(dY, n["y"]), V=(V, n["dV"]), dV=(dV, n["dV"]), dw=(dw, n["lookups"]),
          n_touched=(n_touched, 1))
    _check(_invoke("pkm_stage_value_grad_grouped", h, T, _ptr(w), _ptr(dY), _ptr(V), _ptr(dV), _ptr(dw),
                   _ptr(n_touched), _ptr(ws), _nbytes(ws)), "pkm_stage_value_grad_grouped")


def pkm_stage_value_adam_grouped(h, T, w, dY, V, adam_m, adam_v, adam: dict, dw, n_touched, ws):
    _dt(adam_m, torch.float32, "adam_m")
    _dt(adam_v, torch.float32, "adam_v")
    n = _dims(h, T)
    _need(w=(w, n["lookups"]), dY=(dY, n["y"]), V=(V, n["dV"]), adam_m=(adam_m, n["dV"]), adam_v=(adam_v, n["dV"]),
          dw=(dw, n["lookups"]), n_touched=(n_touched, 1))
    hp = _adam_struct(adam)
    _check(_invoke("pkm_stage_value_adam_grouped", h, T, _ptr(w), _ptr(dY), _ptr(V), _ptr(adam_m), _ptr(adam_v),
                   ctypes.byref(hp), _ptr(dw), _ptr(n_touched), _ptr(ws), _nbytes(ws)),
           "pkm_stage_value_adam_grouped")


def pkm_diagnostics(h, T, idx, w, hits_c, hits_cp, used, entropy, entropy_sum, ws):
    """Monitoring signals of a selection: sub-key hit counts, slots in use, softmax entropy (see pkm.h)."""
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _dt(hits_c, torch.int32, "hits_c")
    _dt(hits_cp, torch.int32, "hits_cp")
    _dt(used, torch.int64, "used")
    _dt(entropy, torch.float32, "entropy")
    _dt(entropy_sum, torch.float64, "entropy_sum")
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), hits_c=(hits_c, n["hits_c"]), hits_cp=(hits_cp, n["hits_cp"]),
          used=(used, n["used"]), entropy=(entropy, n["th"]), entropy_sum=(entropy_sum, 1))
    _check(_invoke("pkm_diagnostics", h, T, _ptr(idx), _ptr(w), _ptr(hits_c), _ptr(hits_cp), _ptr(used),
                   _ptr(entropy), _ptr(entropy_sum), _ptr(ws), _nbytes(ws)), "pkm_diagnostics")


def pkm_stage_subkey_grad(h, T, idx, w, dw, q, C, Cp, dq, dC, dCp, ws):
    n = _dims(h, T)
    _need(idx=(idx, n["lookups"]), w=(w, n["lookups"]), dw=(dw, n["lookups"]), q=(q, n["q"]), C=(C, n["C"]),
          Cp=(Cp, n["Cp"]), dq=(dq, n["q"]), dC=(dC, n["C"]), dCp=(dCp, n["Cp"]))
    _check(_invoke("pkm_stage_subkey_grad", h, T, _ptr(idx), _ptr(w), _ptr(dw), _ptr(q), _ptr(C),
                                       _ptr(Cp), _ptr(dq), _ptr(dC), _ptr(dCp), _ptr(ws), _nbytes(ws)),
           "pkm_stage_subkey_grad")


def pkm_stage_query_grad(h, T, dq, x, Wq, bn_gamma, saved: dict, dWq, dgamma, dbeta, dx, ws):
    n = _dims(h, T)
    _need(dq=(dq, n["q"]), x=(x, n["x"]), Wq=(Wq, n["Wq"]), bn_gamma=(bn_gamma, n["F"]), dWq=(dWq, n["Wq"]),
          dgamma=(dgamma, n["F"]), dbeta=(dbeta, n["F"]), dx=(dx, n["x"]),
          **{"saved['q_pre']": (saved.get("q_pre"), n["q"])},
          **({"saved['bn_mean']": (saved.get("bn_mean"), n["F"]), "saved['bn_rstd']": (saved.get("bn_rstd"), n["F"])}
             if h.cfg.bn == PKM_BN_BATCH else {}))
    sv = _saved_struct(saved)
    _check(_invoke("pkm_stage_query_grad", h, T, _ptr(dq), _ptr(x), _ptr(Wq), _ptr(bn_gamma),
                                      ctypes.byref(sv), _ptr(dWq), _ptr(dgamma), _ptr(dbeta), _ptr(dx), _ptr(ws),
                                      _nbytes(ws)), "pkm_stage_query_grad")


def _need_fwpkm(h, T, streams, q, C, Cp, V, target, y, idx, w):
    """q [T, h*dq], C, Cp, V [streams*|C|*|C'|, d_value], target and y [T, d_value], idx and w [T, h, k]."""
    if int(streams) < 1:
        raise ValueError(f"streams = {streams} < 1")
    n = _dims(h, T, int(streams))
    _need(q=(q, n["q"]), C=(C, n["C"]), Cp=(Cp, n["Cp"]), V=(V, n["V"]), target=(target, n["y"]), y=(y, n["y"]),
          idx=(idx, n["lookups"]), w=(w, n["lookups"]))


def pkm_fwpkm_chunk(h, T, q, C, Cp, V, target, lr, y, idx, w, ws, streams=1):
    """One FwPKM memorization chunk of each of ``streams`` streams (pkm.h): select with IDW scores, y from
    V before the write, then V[r] -= lr * sum w (y - target) over the lookups of each selected row (V
    updated in place; stream b owns the b-th block of |C|*|C'| rows of V and the b-th block of T/streams
    tokens)."""
    st = h.storage
    for n, t in (("q", q), ("C", C), ("Cp", Cp), ("V", V), ("target", target), ("y", y)):
        _dt(t, st, n)
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _need_fwpkm(h, T, streams, q, C, Cp, V, target, y, idx, w)
    _check(_invoke("pkm_fwpkm_chunk", h, T, int(streams), _ptr(q), _ptr(C), _ptr(Cp), _ptr(V), _ptr(target),
                   float(lr), _ptr(y), _ptr(idx), _ptr(w), _ptr(ws), _nbytes(ws)), "pkm_fwpkm_chunk")


def pkm_fwpkm_chunks(h, T, call_T, q, C, Cp, V, target, lr, y, idx, w, ws, streams=1):
    """pkm_fwpkm_chunk on the consecutive slices of ``call_T`` tokens, in order, in one call (pkm.h): the
    selection of all T tokens first (it does not read V), then each slice's gather and value step."""
    st = h.storage
    for n, t in (("q", q), ("C", C), ("Cp", Cp), ("V", V), ("target", target), ("y", y)):
        _dt(t, st, n)
    _dt(idx, torch.int32, "idx")
    _dt(w, torch.float32, "w")
    _need_fwpkm(h, T, streams, q, C, Cp, V, target, y, idx, w)
    _check(_invoke("pkm_fwpkm_chunks", h, T, int(call_T), int(streams), _ptr(q), _ptr(C), _ptr(Cp), _ptr(V),
                   _ptr(target), float(lr), _ptr(y), _ptr(idx), _ptr(w), _ptr(ws), _nbytes(ws)), "pkm_fwpkm_chunks")
