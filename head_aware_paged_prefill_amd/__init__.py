"""SegPagedAttention prefill for AMD MI355X (gfx950): a C-ABI library (librk_seg.so) plus a thin binding.

The library keeps a KV cache paged per (layer, KV head, sequence): GLOBAL heads hold and read every
context page, LOCAL heads only sink plus recent-window pages, and attention runs without a mask.
`rk_seg` mirrors the C entry points; `runner` drives one prefill call of a synthetic workload.
"""
from . import rk_seg  # noqa: F401
from .rk_seg import (RK_BF16, RK_F32, RK_GLOBAL, RK_LOCAL, RkError, load, rk_last_error,  # noqa: F401
                     rk_seg_append_kv, rk_seg_attn_decode, rk_seg_attn_decode_noalloc, rk_seg_attn_prefill,
                     rk_seg_build_tables, rk_seg_key_mass, rk_seg_pack_ledger, rk_seg_pack_pages,
                     rk_seg_pool_create, rk_seg_pool_destroy, rk_seg_pool_free_list, rk_seg_pool_query,
                     rk_seg_reuse_rerotate, rk_seg_tables_advance, rk_seg_tables_advance_workspace_bytes,
                     rk_seg_tables_decode_schedule, rk_seg_tables_destroy, rk_seg_tables_export,
                     rk_seg_tables_mass_schedule, rk_seg_tables_schedule, rk_seg_tables_stats, rk_seg_tables_trim,
                     rk_seg_tables_workspace_bytes, rk_seg_unpack_pages, rk_seg_version, rk_status_string)
