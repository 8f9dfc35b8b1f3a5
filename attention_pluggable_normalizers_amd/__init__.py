"""MI355X-native attention forward with pluggable normalizers.

The compute lives in ``libattn.so`` (HIP kernels for gfx950 behind the C ABI
of ``include/attn.h``); this package is its thin ctypes binding.
"""

from .binding import (
    ATTN_E_INVALID,
    ATTN_E_LAUNCH,
    ATTN_E_UNSUPPORTED,
    ATTN_E_WORKSPACE,
    ATTN_OK,
    NORMALIZER_IDS,
    PATH_NAMES,
    AttnError,
    attn_abi_version,
    attn_bwd,
    attn_bwd_path,
    attn_bwd_varlen,
    attn_fwd,
    attn_fwd_noalloc,
    attn_fwd_path,
    attn_fwd_varlen,
    attn_fwd_workspace_bytes,
    attn_last_error_detail,
    attn_strerror,
    custom_attention,
    load_library,
)

__all__ = [
    "ATTN_OK",
    "ATTN_E_INVALID",
    "ATTN_E_UNSUPPORTED",
    "ATTN_E_WORKSPACE",
    "ATTN_E_LAUNCH",
    "NORMALIZER_IDS",
    "PATH_NAMES",
    "AttnError",
    "attn_abi_version",
    "attn_bwd",
    "attn_bwd_path",
    "attn_bwd_varlen",
    "attn_fwd",
    "attn_fwd_noalloc",
    "attn_fwd_path",
    "attn_fwd_varlen",
    "attn_fwd_workspace_bytes",
    "attn_last_error_detail",
    "attn_strerror",
    "custom_attention",
    "load_library",
]
