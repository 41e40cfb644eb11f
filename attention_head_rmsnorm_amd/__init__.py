"""Flint sink-aware attention (prefill forward and backward, decode) for AMD Instinct MI355X.

The compute path is the HIP library ``libflint_attn.so`` (C ABI in
``include/flint_attn.h``); this package only binds it.
"""

from .binding import (  # noqa: F401
    EXPORTED,
    FLINT_DEV_CACHE,
    KVCache,
    FLINT_ERR_ALIGN,
    FLINT_ERR_DEVICE_DATA,
    FLINT_ERR_HIP,
    FLINT_ERR_NULL,
    FLINT_ERR_SHAPE,
    FLINT_ERR_UNSUPPORTED,
    FLINT_ERR_VALUE,
    FLINT_ERR_WORKSPACE,
    FLINT_OK,
    FLINT_PHASE_ALL,
    FLINT_PHASE_ATTEND,
    FLINT_PHASE_KV,
    FLINT_PHASE_SCHEDULE,
    FlintError,
    flint_attn,
    flint_attn_backward,
    flint_attn_bwd,
    flint_attn_bwd_workspace_bytes,
    flint_attn_fwd_lse,
    flint_attn_decode,
    flint_attn_decode_workspace_bytes,
    flint_attn_device_status,
    flint_attn_fwd,
    flint_attn_fwd_phases,
    flint_attn_kv_append,
    flint_attn_seqused_from_mask,
    flint_attn_strerror,
    flint_attn_workspace_bytes,
    library_path,
    load_library,
    seqused_from_mask,
)
