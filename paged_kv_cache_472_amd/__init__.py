"""MI355X-native paged decode attention and GrowPage page-boundary KV budgeting.

The compute lives in the gfx950 HIP library ``_lib/libgrowpage.so`` (C ABI:
include/growpage.h); :mod:`.growpage` is its ctypes binding.
"""
from .growpage import (  # noqa: F401
    KVCache,
    gp_compact_or_grow,
    gp_compact_or_grow_layers,
    gp_compact_or_grow_layers_workspace_size,
    gp_compact_or_grow_workspace_size,
    gp_paged_decode_attn,
    gp_paged_decode_attn_ex,
    gp_paged_decode_attn_noalloc,
    gp_paged_decode_attn_workspace_size,
    gp_quantize_pages_int4,
    gp_score_and_working_set,
    gp_score_and_working_set_workspace_size,
    gp_update_query_summaries,
    lib,
)
