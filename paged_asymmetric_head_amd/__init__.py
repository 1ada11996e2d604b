"""Paged attention for models whose key and value head dims differ (QK 192, V 128).

The compute path is the HIP library `libdiffkv_attn.so` (hand-written gfx950
kernels behind a C ABI); this package only marshals arguments to it.
Importing the package loads nothing: the library is opened on first use, and
a missing library is an error, never a fallback.
"""

from .binding import (  # noqa: F401
    AttnDesc, DiffKVError, diffkv_attn_decode, diffkv_attn_verify, diffkv_attn_prefill,
    diffkv_attn_mixed, diffkv_attn_partial, diffkv_attn_combine,
    diffkv_attn_workspace_bytes, diffkv_attn_validate, diffkv_attn_strerror, diffkv_attn_num_splits,
    set_profile_events, select_library, diffkv_attn_debug_flags, diffkv_attn_timeline_buffer, prepared_call,
    diffkv_kv_write, prepared_kv_write,
    library_path,
    load_library,
)
