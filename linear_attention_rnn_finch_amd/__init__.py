"""Finch WKV pre-fill on MI355X (gfx950).

The hot path of GoldFinch's linear-time pre-fill -- the Finch (RWKV-6) WKV
recurrence with per-channel data-dependent decay -- as hand-written HIP kernels
behind a C ABI (include/finch_wkv.h, libfinch_wkv.so).  This package is the
thin Python binding over that library.
"""
from ._binding import (  # noqa: F401
    HEAD_DIM, LIBRARY_PATH, WORKSPACE_CONTROL_BYTES, WkvError, abi_version, gold_compress,
    layernorm_heads, new_workspace, prefill, prefill_varlen, set_split_launches, set_wait_bound,
    varlen_workspace_bytes, workspace_bytes, workspace_errors)
