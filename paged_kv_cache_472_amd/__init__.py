"""MI355X-native paged decode attention and GrowPage page-boundary KV budgeting.

The compute lives in the gfx950 HIP library ``_lib/libgrowpage.so`` (C ABI:
include/growpage.h); :mod:`.growpage` is its ctypes binding.
"""
from .growpage import (  # noqa: F401
    KVCache,
    gp_compact_or_grow,
    gp_paged_decode_attn,
    gp_score_and_working_set,
    gp_update_query_summaries,
    lib,
)
