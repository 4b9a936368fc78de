"""Product-key memory (PKM) lookup for AMD Instinct MI355X (gfx950).

The work is done by hand-written HIP kernels in ``libpkm.so`` behind the C ABI
of ``include/pkm.h``; this package is its thin Python binding (``_lib``) plus a
convenience layer (``memory``) that allocates the caller-owned buffers with
torch.  PyTorch provides device memory and streams only.
"""
from ._lib import (EXPORTED, PKM_BF16, PKM_BN_BATCH, PKM_BN_NONE, PKM_F32, PKM_SCORE_DOT, PKM_SCORE_IDW,
                   PKM_VALUES_FP8, PKM_VALUES_STORAGE, PKM_WS_BACKWARD, PKM_WS_FORWARD, PKM_WS_FWPKM_CHUNK, Handle,
                   PkmError, lib, make_config, pkm_adam, pkm_adam_rows, pkm_backward, pkm_backward_adam,
                   pkm_backward_adam_rows, pkm_config, pkm_create,
                   pkm_diagnostics, pkm_forward, pkm_forward_noalloc, pkm_fwpkm_chunk, pkm_fwpkm_chunks, pkm_get_config, pkm_quantize_values, pkm_saved,
                   pkm_stage_gather, pkm_stage_merge_softmax, pkm_stage_query, pkm_stage_query_grad,
                   pkm_stage_row_groups, pkm_stage_score_topk, pkm_stage_subkey_grad, pkm_stage_value_adam,
                   pkm_stage_value_adam_grouped, pkm_stage_value_adam_rows, pkm_stage_value_grad, pkm_stage_value_grad_grouped,
                   pkm_workspace_size)
from .memory import ProductKeyMemory

__all__ = [
    "EXPORTED", "Handle", "PkmError", "ProductKeyMemory", "lib", "make_config",
    "pkm_adam", "pkm_adam_rows", "pkm_backward", "pkm_backward_adam", "pkm_backward_adam_rows", "pkm_config", "pkm_create", "pkm_diagnostics", "pkm_forward", "pkm_forward_noalloc",
    "pkm_fwpkm_chunk", "pkm_fwpkm_chunks", "pkm_get_config", "pkm_quantize_values", "pkm_saved", "pkm_stage_gather",
    "pkm_stage_merge_softmax", "pkm_stage_query", "pkm_stage_query_grad", "pkm_stage_row_groups",
    "pkm_stage_score_topk", "pkm_stage_subkey_grad", "pkm_stage_value_adam", "pkm_stage_value_adam_grouped", "pkm_stage_value_adam_rows",
    "pkm_stage_value_grad", "pkm_stage_value_grad_grouped", "pkm_workspace_size",
    "PKM_F32", "PKM_BF16", "PKM_BN_NONE", "PKM_BN_BATCH", "PKM_VALUES_STORAGE", "PKM_VALUES_FP8",
    "PKM_SCORE_DOT", "PKM_SCORE_IDW", "PKM_WS_FORWARD", "PKM_WS_BACKWARD", "PKM_WS_FWPKM_CHUNK",
]
