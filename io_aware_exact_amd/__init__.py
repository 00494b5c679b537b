"""Exact IO-aware attention forward for AMD MI355X (gfx950).

The compute path is the HIP library ``libattn.so`` behind the C ABI declared
in ``include/attn.h``; this package binds it with the same names.
"""

from .attn import (
    ATTN_EHIP,
    ATTN_EINVAL,
    ATTN_EUNSUPPORTED,
    ATTN_EWORKSPACE,
    ATTN_OK,
    AttnError,
    attn_bwd,
    attn_bwd_workspace_bytes,
    attn_decode,
    attn_decode_gqa,
    attn_decode_noalloc,
    attn_decode_noalloc_max_bytes,
    attn_decode_splits,
    attn_decode_workspace_bytes,
    attn_fwd,
    attn_fwd_f32,
    attn_fwd_split,
    attn_fwd_split_workspace_bytes,
    attn_last_kernel,
    attn_status_string,
    lib,
    prepared_bwd,
    prepared_decode,
    prepared_fwd,
)

__all__ = [
    "ATTN_EHIP", "ATTN_EINVAL", "ATTN_EUNSUPPORTED", "ATTN_EWORKSPACE", "ATTN_OK", "AttnError", "attn_bwd",
    "attn_bwd_workspace_bytes", "prepared_bwd",
    "attn_decode", "attn_decode_gqa", "attn_decode_noalloc", "attn_decode_noalloc_max_bytes", "attn_decode_splits",
    "attn_decode_workspace_bytes", "attn_fwd", "attn_fwd_f32",
    "attn_fwd_split", "attn_fwd_split_workspace_bytes", "attn_last_kernel", "attn_status_string", "lib",
    "prepared_decode", "prepared_fwd",
]
