"""Causal kernelized linear attention for AMD Instinct MI355X (gfx950).

The computation runs in hand-written HIP kernels behind the C ABI of
``liblinattn.so`` (include/linattn.h); this package is its thin Python binding
(``forward``, ``decode_step``, ``featmap``) plus the seeded input generators in
``inputs``.  Build the library with ``python -m kernelized_attention_scan_amd.build``.
"""
from ._binding import (LA_BF16, LA_F32, LIB_PATH, MAP_ELU1, MAP_IDENTITY,
                       MAP_PERFORMER, SYMBOLS, LinAttnError, cached_workspace,
                       backward, backward_workspace_bytes, decode_step,
                       decode_step_gated, featmap,
                       forward, forward_train,
                       forward_gated, forward_noalloc,
                       forward_workspace_bytes, gated_workspace_bytes,
                       linear_attention,
                       load_library, new_workspace, set_exchange_spin_limit,
                       workspace_check)

__all__ = ["forward", "forward_train", "backward", "backward_workspace_bytes",
           "linear_attention",
           "forward_gated", "forward_noalloc", "decode_step",
           "decode_step_gated", "featmap", "forward_workspace_bytes",
           "gated_workspace_bytes",
           "new_workspace", "workspace_check", "cached_workspace",
           "set_exchange_spin_limit",
           "load_library", "LinAttnError", "LIB_PATH", "SYMBOLS", "MAP_IDENTITY",
           "MAP_ELU1", "MAP_PERFORMER", "LA_F32", "LA_BF16"]
