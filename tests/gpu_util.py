"""Helpers for the GPU tests: seeded numpy inputs -> torch device tensors."""
from __future__ import annotations

import os
import sys

import numpy as np
import torch

import pkm_inputs as pi


def note(msg: str) -> None:
    """Name the case on stdout before GPU work, so a failed run says which case it was."""
    print(msg, flush=True)
    sys.stdout.flush()


def storage_dtype(dtype: str) -> torch.dtype:
    return torch.bfloat16 if dtype == "bf16" else torch.float32


def to_dev(a: np.ndarray, dtype: str | None = None) -> torch.Tensor:
    """numpy -> cuda tensor; uint16 arrays are bf16 bit patterns."""
    if a.dtype == np.uint16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a))
    return t.cuda()


def layer_for(cfg, accumulate_dv=True, values="storage", score="dot"):
    from product_key_memory_pkm_amd import ProductKeyMemory
    return ProductKeyMemory(cfg.d, cfg.heads, cfg.dq, cfg.n_keys, cfg.n_keys2, cfg.topk, cfg.d_value,
                            dtype=cfg.dtype, bn=cfg.bn, bn_eps=cfg.bn_eps, temperature=cfg.temperature,
                            accumulate_dv=accumulate_dv, values=values, score=score)


def fp8_table(scale: np.ndarray, codes: np.ndarray) -> np.ndarray:
    """Bytes of an fp8 value table (pkm.h, PKM_VALUES_FP8): per row a 16-byte header holding the fp32 scale
    (other bytes zero), then the row's E4M3 codes, then zeros up to d + 16 rounded up to 128 bytes."""
    n, d = codes.shape
    out = np.zeros((n, (d + 16 + 127) // 128 * 128), dtype=np.uint8)
    out[:, :4] = np.asarray(scale, dtype=np.float32).reshape(n, 1).view(np.uint8)
    out[:, 16:16 + d] = codes
    return out.reshape(-1)


def upload(inp: dict) -> dict:
    return {k: to_dev(v) for k, v in inp.items() if isinstance(v, np.ndarray) and k != "mixture_labels"}


def require_lib():
    from product_key_memory_pkm_amd import lib
    lib()   # raises if libpkm.so is missing
    if not torch.cuda.is_available():
        raise RuntimeError("no GPU visible")
