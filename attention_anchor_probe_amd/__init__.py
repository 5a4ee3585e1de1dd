"""MI355X-native slot-mapped bidirectional attention engine for the ACache
affix cache ("Affix Cache for Diffusion Large Language Models").

The path runs in libacache.so (hand-written HIP kernels for gfx950, C ABI in
include/acache.h); this package only binds it.
"""
from .binding import (  # noqa: F401
    AcacheError, KVPool, MapArgs, EXPORTS, LIB_PATH, make_pool, map_args,
    acache_version, acache_anchor_count, acache_probe_workspace_bytes, acache_probe_scores,
    acache_probe_attention, acache_probe_column_mass_workspace_bytes, acache_probe_column_mass,
    acache_topk_anchors, acache_build_maps, acache_scatter_private, acache_block_slots,
    acache_mapped_attention, acache_mapped_attention_shared_workspace_bytes, acache_mapped_attention_shared,
    acache_mapped_attention_shared_noalloc,
    acache_store_attend_workspace_bytes, acache_store_attend,
    acache_hkvd_scores, acache_lse_merge, acache_kv_footprint, acache_validate_slots,
    ACACHE_CHECK_READ, ACACHE_CHECK_WRITE, acache_check_slots, acache_scatter_private_checked,
)
