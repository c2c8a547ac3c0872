"""Kascade cross-layer Top-k sparse attention on MI355X (gfx950).

Thin Python binding over the C ABI in include/kascade.h (libkascade_mi355x.so).
Every computation runs in the HIP library; this module only marshals torch
tensors (device memory) and the current HIP stream into the C calls. There is
no CPU or PyTorch fallback: if the library is missing, importing the binding
raises.
"""
from .binding import (  # noqa: F401
    KasError,
    decode_anchor,
    decode_dense,
    decode_k,
    decode_refine,
    decode_reuse,
    decode_reuse_noalloc,
    NOALLOC_SCRATCH_BYTES,
    lib_path,
    make_desc,
    prefill_anchor,
    prefill_dense,
    prefill_offsets,
    prefill_reuse,
    profile_enable,
    profile_names,
    profile_query,
    profile_reset,
    topk_count,
    workspace_size,
    set_option,
    get_option,
    OPT_DECODE_SPLIT_ROWS,
    OPT_DECODE_SELECT_ONE_PASS,
    OPT_PREFILL_POOL_MB,
    OPT_PREFILL_SELECT_CAP,
    OP_DECODE_ANCHOR,
    OP_DECODE_REUSE,
    OP_PREFILL_ANCHOR,
    OP_PREFILL_REUSE,
    OP_DECODE_DENSE,
    OP_PREFILL_DENSE,
)
from .binding import _load as _load_library

# Fail loudly at import when the HIP library is missing: there is no fallback.
_load_library()
