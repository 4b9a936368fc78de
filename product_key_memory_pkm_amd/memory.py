"""Convenience wrapper: allocates the caller-owned buffers of the C ABI with torch.

Nothing here computes: ``forward`` / ``backward`` allocate outputs, saved state
and workspace, then call ``pkm_forward`` / ``pkm_backward``.
"""
from __future__ import annotations

import torch

from . import _lib as L


class ProductKeyMemory:
    """Product-key memory layer shape + handle.

    Parameters follow the C ABI (``pkm_config``): input width ``d_in``, ``heads``,
    per-head query width ``d_query``, codebook sizes ``n_keys`` / ``n_keys2``,
    ``topk``, value width ``d_value``, storage dtype ``"f32"`` or ``"bf16"``, value table format ``values``
    (``"storage"`` or ``"fp8"``: rows of a fp32 scale and E4M3 codes, forward only), sub-key score
    ``score`` (``"dot"``, or ``"idw"``: -log of the Euclidean distance, as the fast-weight memory scores;
    forward and ``fwpkm_chunk`` only).
    """

    def __init__(self, d_in, heads, d_query, n_keys, n_keys2, topk, d_value, dtype="bf16", bn=True, bn_eps=1e-5,
                 temperature=1.0, accumulate_dv=True, device="cuda", values="storage", score="dot"):
        self.cfg = L.make_config(d_in, heads, d_query, n_keys, n_keys2, topk, d_value, dtype, bn, bn_eps,
                                 temperature, accumulate_dv, values, score)
        self.handle = L.pkm_create(self.cfg)
        self.device = torch.device(device)
        self._ws = None

    @property
    def storage(self) -> torch.dtype:
        return self.handle.storage

    def workspace(self, T: int, with_backward) -> torch.Tensor:
        n = L.pkm_workspace_size(self.handle, T, with_backward)
        if self._ws is None or self._ws.numel() < n:
            self._ws = torch.empty(max(n, 256), dtype=torch.uint8, device=self.device)
        return self._ws

    def alloc_saved(self, T: int) -> dict:
        c = self.cfg
        F = c.heads * c.d_query
        dev = self.device
        sv = {"idx": torch.empty((T, c.heads, c.topk), dtype=torch.int32, device=dev),
              "w": torch.empty((T, c.heads, c.topk), dtype=torch.float32, device=dev),
              "q": torch.empty((T, F), dtype=self.storage, device=dev),
              "q_pre": torch.empty((T, F), dtype=torch.float32, device=dev)}
        if c.bn:
            sv["bn_mean"] = torch.empty(F, dtype=torch.float32, device=dev)
            sv["bn_rstd"] = torch.empty(F, dtype=torch.float32, device=dev)
        return sv

    def quantize_values(self, V):
        """fp8 value table of V [rows, d_value]: uint8 bytes, rows of a fp32 scale header and E4M3 codes padded
        to whole 128-byte lines (fp8_row_bytes(d_value) bytes each)."""
        out = torch.empty(V.shape[0] * L.fp8_row_bytes(self.cfg.d_value), dtype=torch.uint8, device=self.device)
        L.pkm_quantize_values(self.handle, V, out)
        return out

    def forward(self, x, Wq, gamma, beta, C, Cp, V, saved=None, y=None):
        T = x.shape[0]
        saved = saved if saved is not None else self.alloc_saved(T)
        y = y if y is not None else torch.empty((T, self.cfg.d_value), dtype=self.storage, device=self.device)
        ws = self.workspace(T, False)
        L.pkm_forward(self.handle, T, x, Wq, gamma, beta, C, Cp, V, y, saved, ws)
        return y, saved

    def backward(self, dY, x, Wq, gamma, C, Cp, V, saved, dV, want_dx=True, out=None):
        c = self.cfg
        T = x.shape[0]
        F = c.heads * c.d_query
        dev = self.device
        g = out if out is not None else {
            "touched": torch.empty(max(1, T * c.heads * c.topk), dtype=torch.int32, device=dev),
            "n_touched": torch.zeros(1, dtype=torch.int64, device=dev),
            "dC": torch.empty((c.heads, c.n_keys, c.d_query // 2), dtype=torch.float32, device=dev),
            "dCp": torch.empty((c.heads, c.n_keys2, c.d_query // 2), dtype=torch.float32, device=dev),
            "dWq": torch.empty((F, c.d_in), dtype=torch.float32, device=dev),
            "dgamma": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dbeta": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dx": torch.empty((T, c.d_in), dtype=self.storage, device=dev) if want_dx else None,
        }
        ws = self.workspace(T, True)
        L.pkm_backward(self.handle, T, dY, x, Wq, gamma, C, Cp, V, saved, dV, g["touched"], g["n_touched"], g["dC"],
                       g["dCp"], g["dWq"], g["dgamma"], g["dbeta"], g["dx"], ws)
        return g

    def backward_adam(self, dY, x, Wq, gamma, C, Cp, V, saved, adam_m, adam_v, adam: dict, want_dx=True, out=None):
        """Backward with the Adam step of the touched value rows fused in (V, adam_m, adam_v updated in place).

        ``adam``: {"lr", "beta1", "beta2", "eps", "step"} (step counts from 1).  Returns the other gradients."""
        c = self.cfg
        T = x.shape[0]
        F = c.heads * c.d_query
        dev = self.device
        g = out if out is not None else {
            "touched": torch.empty(max(1, T * c.heads * c.topk), dtype=torch.int32, device=dev),
            "n_touched": torch.zeros(1, dtype=torch.int64, device=dev),
            "dC": torch.empty((c.heads, c.n_keys, c.d_query // 2), dtype=torch.float32, device=dev),
            "dCp": torch.empty((c.heads, c.n_keys2, c.d_query // 2), dtype=torch.float32, device=dev),
            "dWq": torch.empty((F, c.d_in), dtype=torch.float32, device=dev),
            "dgamma": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dbeta": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dx": torch.empty((T, c.d_in), dtype=self.storage, device=dev) if want_dx else None,
        }
        ws = self.workspace(T, True)
        L.pkm_backward_adam(self.handle, T, dY, x, Wq, gamma, C, Cp, V, saved, adam_m, adam_v, adam, g["touched"],
                            g["n_touched"], g["dC"], g["dCp"], g["dWq"], g["dgamma"], g["dbeta"], g["dx"], ws)
        return g

    def adam_row_state(self, capacity: int) -> dict:
        """Moment pool for ``backward_adam_rows``: ``capacity`` rows of first and second moments, handed
        out to value rows on their first gradient (slot -1: none yet; n_used: slots handed out)."""
        c = self.cfg
        dev = self.device
        return {"slot": torch.full((c.n_keys * c.n_keys2,), -1, dtype=torch.int32, device=dev),
                "m": torch.empty((capacity, c.d_value), dtype=torch.float32, device=dev),
                "v": torch.empty((capacity, c.d_value), dtype=torch.float32, device=dev),
                "n_used": torch.zeros(1, dtype=torch.int64, device=dev)}

    def backward_adam_rows(self, dY, x, Wq, gamma, C, Cp, V, saved, state: dict, adam: dict, want_dx=True):
        """``backward_adam`` with the moments in a pool of slots (``adam_row_state``).  A touched row that
        finds the pool full is not stepped; ``state["n_used"]`` above the capacity reports that."""
        c = self.cfg
        T = x.shape[0]
        F = c.heads * c.d_query
        dev = self.device
        g = {
            "touched": torch.empty(max(1, T * c.heads * c.topk), dtype=torch.int32, device=dev),
            "n_touched": torch.zeros(1, dtype=torch.int64, device=dev),
            "dC": torch.empty((c.heads, c.n_keys, c.d_query // 2), dtype=torch.float32, device=dev),
            "dCp": torch.empty((c.heads, c.n_keys2, c.d_query // 2), dtype=torch.float32, device=dev),
            "dWq": torch.empty((F, c.d_in), dtype=torch.float32, device=dev),
            "dgamma": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dbeta": torch.empty(F, dtype=torch.float32, device=dev) if c.bn else None,
            "dx": torch.empty((T, c.d_in), dtype=self.storage, device=dev) if want_dx else None,
        }
        ws = self.workspace(T, True)
        L.pkm_backward_adam_rows(self.handle, T, dY, x, Wq, gamma, C, Cp, V, saved, state, adam, g["touched"],
                                 g["n_touched"], g["dC"], g["dCp"], g["dWq"], g["dgamma"], g["dbeta"], g["dx"], ws)
        return g

    def fwpkm_chunk(self, q, C, Cp, V, target, lr: float, out=None, streams: int = 1):
        """One memorization chunk of the fast-weight memory (``pkm_fwpkm_chunk``) for each of ``streams``
        streams: returns (y, idx, w), y read from V before the write; V is updated in place."""
        T = q.shape[0]
        c = self.cfg
        dev = self.device
        if out is None:
            out = {"y": torch.empty((T, c.d_value), dtype=self.storage, device=dev),
                   "idx": torch.empty((T, c.heads, c.topk), dtype=torch.int32, device=dev),
                   "w": torch.empty((T, c.heads, c.topk), dtype=torch.float32, device=dev)}
        ws = self.workspace(T, L.PKM_WS_FWPKM_CHUNK)
        L.pkm_fwpkm_chunk(self.handle, T, q, C, Cp, V, target, lr, out["y"], out["idx"], out["w"], ws, streams)
        return out["y"], out["idx"], out["w"]

    def fwpkm_chunks(self, q, C, Cp, V, target, lr: float, call_T: int, out=None, streams: int = 1):
        """``fwpkm_chunk`` on the consecutive slices of ``call_T`` tokens of q and target, in order, in one call
        (``pkm_fwpkm_chunks``): returns (y, idx, w) for all tokens; V is updated in place."""
        T = q.shape[0]
        c = self.cfg
        dev = self.device
        if out is None:
            out = {"y": torch.empty((T, c.d_value), dtype=self.storage, device=dev),
                   "idx": torch.empty((T, c.heads, c.topk), dtype=torch.int32, device=dev),
                   "w": torch.empty((T, c.heads, c.topk), dtype=torch.float32, device=dev)}
        ws = self.workspace(T, L.PKM_WS_FWPKM_CHUNK)
        L.pkm_fwpkm_chunks(self.handle, T, call_T, q, C, Cp, V, target, lr, out["y"], out["idx"], out["w"], ws,
                           streams)
        return out["y"], out["idx"], out["w"]
