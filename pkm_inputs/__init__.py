"""Seeded synthetic inputs for the product-key memory lookup.

This module only draws random numbers and encodes them; it holds none of the
lookup's arithmetic.  Both the CPU oracle (``oracle/``) and the HIP path (via
the tests and ``bench.py``) take their inputs from here, so the two sides see
identical bits.

Generator: numpy ``PCG64``.  Every tensor is split into fixed chunks of
``CHUNK`` elements; chunk ``c`` of tensor ``n`` (``n`` is the tensor's position
in the fixed draw order below) is drawn from
``PCG64(SeedSequence(seed, spawn_key=(n, c)))``.  The bits therefore do not
depend on how many threads fill the tensor.

Draw order: x, W_q, C, C', V, dY (the Gaussian-mixture tokens of the skewed
workload are part of x: centroids, labels, then noise).

bf16 tensors are produced as fp32 draws rounded to the nearest bf16
(ties to even) and returned as ``uint16`` bit patterns.

Workloads (shapes and distributions of the memory layer the pages describe:
the product-key memory paper's summary gives h=4 heads, k=32 and 512^2-1024^2
slots for a 1600-dim model; the blog's simplified layer fixes a bias-free
query projection and two half-dim sub-key codebooks):

=========  ======  =====  ==  ===  ====  =========  ==  =====  ====
name       T       d      h   dq   |C|   slots      k   dtype  BN
=========  ======  =====  ==  ===  ====  =========  ==  =====  ====
tiny       64      64     1   32   32    1,024      8   f32    off
small      8192    512    4   256  256   65,536     32  f32    batch
paper      32768   1600   4   512  1024  1,048,576  32  bf16   batch
skewed     65536   1024   8   512  2048  4,194,304  32  bf16   batch
=========  ======  =====  ==  ===  ====  =========  ==  =====  ====

``paper_bwd`` is ``paper`` plus an upstream gradient dY; ``skewed`` draws its
tokens from a 256-centroid Gaussian mixture with Zipf(1) mixture weights so
that slot access is skewed.
"""
from __future__ import annotations

import math
import os
from concurrent.futures import ThreadPoolExecutor
from dataclasses import dataclass, field, replace

import numpy as np

CHUNK = 1 << 22

F32 = "f32"
BF16 = "bf16"


# --------------------------------------------------------------------------
# bf16 encoding (storage format only)
# --------------------------------------------------------------------------
def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 values to the nearest bf16 (ties to even); return uint16 bits."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32)
    r = (u + np.uint32(0x7FFF) + ((u >> np.uint32(16)) & np.uint32(1))) >> np.uint32(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(b: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


# --------------------------------------------------------------------------
# chunked, thread-count-independent draws
# --------------------------------------------------------------------------
def _threads() -> int:
    n = os.cpu_count() or 1
    return max(1, min(16, n))


def _fill(seed: int, tensor_id: int, n: int, kind: str, a: float, b: float, dtype: str = F32) -> np.ndarray:
    """n fp32 draws (chunk c from its own stream), or their bf16 bits when dtype is bf16.

    The bf16 case rounds chunk by chunk, so large tensors never exist in fp32.
    """
    out = np.empty(n, dtype=np.uint16 if dtype == BF16 else np.float32)
    nchunks = (n + CHUNK - 1) // CHUNK

    def work(c: int) -> None:
        g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(tensor_id, c))))
        lo, hi = c * CHUNK, min(n, (c + 1) * CHUNK)
        view = out[lo:hi] if dtype != BF16 else np.empty(hi - lo, dtype=np.float32)
        if kind == "normal":
            g.standard_normal(out=view, dtype=np.float32)
            if a != 0.0 or b != 1.0:
                view *= np.float32(b)
                view += np.float32(a)
        elif kind == "uniform":
            g.random(out=view, dtype=np.float32)
            view *= np.float32(b - a)
            view += np.float32(a)
        elif kind == "int":
            view[:] = g.integers(int(a), int(b) + 1, size=hi - lo).astype(np.float32)
        else:
            raise ValueError(kind)
        if dtype == BF16:
            out[lo:hi] = f32_to_bf16_bits(view)

    if nchunks == 1:
        work(0)
    else:
        with ThreadPoolExecutor(_threads()) as ex:
            list(ex.map(work, range(nchunks)))
    return out


def _encode(a: np.ndarray, dtype: str) -> np.ndarray:
    return f32_to_bf16_bits(a) if dtype == BF16 else a


# --------------------------------------------------------------------------
# configurations
# --------------------------------------------------------------------------
@dataclass(frozen=True)
class Config:
    name: str
    T: int
    d: int
    heads: int
    dq: int
    n_keys: int
    n_keys2: int
    topk: int
    d_value: int
    dtype: str
    bn: bool
    seed: int
    bn_eps: float = 1e-5
    temperature: float = 1.0
    x_kind: str = "normal"          # "normal" | "mixture" | "int"
    wq_kind: str = "glorot"         # "glorot" | "int"
    key_kind: str = "uniform"       # "uniform" (+-1/sqrt(dq/2)) | "int"
    v_std: float = 0.0              # 0 -> d_value**-0.5
    int_range: int = 3
    mixture: dict = field(default_factory=dict)

    @property
    def slots(self) -> int:
        return self.n_keys * self.n_keys2

    @property
    def F(self) -> int:
        return self.heads * self.dq


CONFIGS = {
    "tiny": Config("tiny", T=64, d=64, heads=1, dq=32, n_keys=32, n_keys2=32, topk=8, d_value=64,
                   dtype=F32, bn=False, seed=0, v_std=0.05),
    "small": Config("small", T=8192, d=512, heads=4, dq=256, n_keys=256, n_keys2=256, topk=32,
                    d_value=512, dtype=F32, bn=True, seed=1),
    "paper": Config("paper", T=32768, d=1600, heads=4, dq=512, n_keys=1024, n_keys2=1024, topk=32,
                    d_value=1600, dtype=BF16, bn=True, seed=2),
    "skewed": Config("skewed", T=65536, d=1024, heads=8, dq=512, n_keys=2048, n_keys2=2048, topk=32,
                     d_value=1024, dtype=BF16, bn=True, seed=4, x_kind="mixture",
                     mixture={"centroids": 256, "sigma": 0.5, "zipf_s": 1.0}),
}


def custom(**kw) -> Config:
    """A config for tests: fields of ``Config``; ``name`` defaults to 'custom'."""
    kw.setdefault("name", "custom")
    kw.setdefault("n_keys2", kw.get("n_keys"))
    kw.setdefault("d_value", kw.get("d"))
    return Config(**kw)


def with_tokens(cfg: Config, T: int) -> Config:
    return replace(cfg, T=T)


def make_inputs(cfg: Config, with_dy: bool = False) -> dict:
    """Draw x, W_q, C, C', V (and dY) for ``cfg``; bf16 tensors as uint16 bits.

    Shapes: x [T, d]; Wq [h*dq, d] (out x in); C [h, |C|, dq/2]; Cp [h, |C'|, dq/2];
    V [|C|*|C'|, d_value]; dY [T, d_value]; gamma/beta [h*dq] fp32 (1 and 0).
    """
    s = cfg.seed
    T, d, h, dq = cfg.T, cfg.d, cfg.heads, cfg.dq
    half = dq // 2
    ir = float(cfg.int_range)
    out = {}

    # x
    if cfg.x_kind == "normal":
        x = _fill(s, 0, T * d, "normal", 0.0, 1.0)
    elif cfg.x_kind == "int":
        x = _fill(s, 0, T * d, "int", -ir, ir)
    elif cfg.x_kind == "mixture":
        m = cfg.mixture
        nc = int(m["centroids"])
        mu = _fill(s, 100, nc * d, "normal", 0.0, 1.0).reshape(nc, d)
        p = 1.0 / np.arange(1, nc + 1, dtype=np.float64) ** float(m["zipf_s"])
        cdf = np.cumsum(p / p.sum())
        u = _fill(s, 101, T, "uniform", 0.0, 1.0).astype(np.float64)
        z = np.minimum(np.searchsorted(cdf, u, side="right"), nc - 1)
        eps = _fill(s, 102, T * d, "normal", 0.0, float(m["sigma"])).reshape(T, d)
        x = (mu[z] + eps).astype(np.float32).reshape(-1)
        out["mixture_labels"] = z.astype(np.int32)
    else:
        raise ValueError(cfg.x_kind)
    out["x"] = _encode(x.reshape(T, d), cfg.dtype)

    # W_q (Glorot-uniform over fan_in=d, fan_out=h*dq)
    F = h * dq
    if cfg.wq_kind == "glorot":
        lim = math.sqrt(6.0 / (d + F))
        wq = _fill(s, 1, F * d, "uniform", -lim, lim)
    else:
        wq = _fill(s, 1, F * d, "int", -ir, ir)
    out["Wq"] = _encode(wq.reshape(F, d), cfg.dtype)

    # sub-key codebooks
    for tid, name, nk in ((2, "C", cfg.n_keys), (3, "Cp", cfg.n_keys2)):
        if cfg.key_kind == "uniform":
            lim = 1.0 / math.sqrt(half)
            a = _fill(s, tid, h * nk * half, "uniform", -lim, lim)
        else:
            a = _fill(s, tid, h * nk * half, "int", -ir, ir)
        out[name] = _encode(a.reshape(h, nk, half), cfg.dtype)

    # values
    K = cfg.slots
    if cfg.x_kind == "int" and cfg.key_kind == "int":
        v = _fill(s, 4, K * cfg.d_value, "int", -ir, ir, cfg.dtype)
    else:
        std = cfg.v_std if cfg.v_std > 0 else cfg.d_value ** -0.5
        v = _fill(s, 4, K * cfg.d_value, "normal", 0.0, std, cfg.dtype)
    out["V"] = v.reshape(K, cfg.d_value)

    if with_dy:
        dy = _fill(s, 5, T * cfg.d_value, "normal", 0.0, 1.0, cfg.dtype)
        out["dY"] = dy.reshape(T, cfg.d_value)

    out["gamma"] = np.ones(F, dtype=np.float32)
    out["beta"] = np.zeros(F, dtype=np.float32)
    return out


# --------------------------------------------------------------------------
# inputs for single-stage tests
# --------------------------------------------------------------------------
def random_selection(seed: int, T: int, heads: int, k: int, n_rows: int, zipf: float = 0.0):
    """Random (row, weight) lists [T, h, k] plus a stage-test dY seed.

    Rows are drawn uniformly (or Zipf-like when ``zipf`` > 0) and may repeat
    within a list; weights are positive and sum to 1 per (t, h).
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(200,))))
    if zipf > 0:
        ranks = np.arange(1, n_rows + 1, dtype=np.float64)
        p = ranks ** -zipf
        cdf = np.cumsum(p / p.sum())
        u = g.random(T * heads * k)
        perm = g.permutation(n_rows)
        rows = perm[np.minimum(np.searchsorted(cdf, u, side="right"), n_rows - 1)]
    else:
        rows = g.integers(0, n_rows, size=T * heads * k)
    w = g.random(T * heads * k).astype(np.float32).reshape(T, heads, k) + np.float32(0.05)
    w = (w / w.sum(axis=-1, keepdims=True)).astype(np.float32)
    return rows.astype(np.int32).reshape(T, heads, k), w


def random_array(seed: int, tag: int, shape, dtype: str = F32, std: float = 1.0) -> np.ndarray:
    n = int(np.prod(shape))
    a = _fill(seed, 300 + tag, n, "normal", 0.0, std).reshape(shape)
    return _encode(a, dtype)


def random_ints(seed: int, tag: int, shape, lo: int, hi: int, dtype: str = F32) -> np.ndarray:
    n = int(np.prod(shape))
    a = _fill(seed, 400 + tag, n, "int", lo, hi).reshape(shape)
    return _encode(a, dtype)


def random_sublists(seed: int, T: int, heads: int, k: int, nk: int, nk2: int, integer: bool = False):
    """Per-half candidate lists [T, h, 2, k]: distinct sub-key ids with fp32 scores.

    Each list is arranged by score descending, then id ascending (the order the
    merge stage expects from the per-half selection).  ``integer`` draws scores
    from a few small integers so that equal scores are common.
    """
    g = np.random.Generator(np.random.PCG64(np.random.SeedSequence(seed, spawn_key=(500,))))
    idx = np.empty((T, heads, 2, k), dtype=np.int32)
    sc = np.empty((T, heads, 2, k), dtype=np.float32)
    for p, n in ((0, nk), (1, nk2)):
        ids = np.argsort(g.random((T * heads, n)), axis=1)[:, :k]
        if integer:
            s = g.integers(-2, 3, size=(T * heads, k)).astype(np.float32)
        else:
            s = g.standard_normal((T * heads, k)).astype(np.float32)
        order = np.lexsort((ids, -s), axis=1)
        idx[:, :, p, :] = np.take_along_axis(ids, order, axis=1).reshape(T, heads, k)
        sc[:, :, p, :] = np.take_along_axis(s, order, axis=1).reshape(T, heads, k)
    return idx, sc


# --------------------------------------------------------------------------
# fast-weight memory (FwPKM) stream
# --------------------------------------------------------------------------
def fwpkm_stream(seed: int, n_tokens: int, width: int, d_value: int, dtype: str = F32):
    """Queries and lookahead targets of one token stream for the fast-weight memory.

    q [n_tokens, width] ~ N(0, 2/width) (each half-query has unit expected norm, like the
    uniform sub-keys); the stream's value vectors v [n_tokens + 1, d_value] ~ N(0, 1) and
    the target of token t is v[t + 1] (the next token's value: the lookahead target of the
    fast-weight page).  Both encoded in ``dtype``.
    """
    q = _fill(seed, 600, n_tokens * width, "normal", 0.0, math.sqrt(2.0 / width))
    v = _fill(seed, 601, (n_tokens + 1) * d_value, "normal", 0.0, 1.0).reshape(n_tokens + 1, d_value)
    return _encode(q.reshape(n_tokens, width), dtype), _encode(np.ascontiguousarray(v[1:]), dtype)
