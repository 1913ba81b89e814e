"""KV-cache sparsification on MI355X: the prefill-and-compress path behind libkvs.

    kvs_prefill_attn_lse -> kvs_window_score -> kvs_topk_select -> kvs_compact_paged -> kvs_paged_decode
    (kvs_topk_compact: the selection and the compaction in one launch)

Every step runs in hand-written HIP kernels for gfx950 (libkvs.so, built in-tree with
``python kv_cache_sparsification_amd/build.py``).  This package only marshals torch tensors
into the C ABI declared in include/kvs.h; importing it fails if the library is not built.
"""
from ._lib import lib, KvsError, BLOCK_SIZE, LIB_PATH
from .ops import (kvs_prefill_attn_lse, kvs_window_score, kvs_topk_select, kvs_compact_paged, kvs_topk_compact,
                  kvs_paged_decode, kvs_paged_decode_workspace_size, kvs_copy_blocks, new_pools,
                  kvs_slot_init, kvs_decode_select_slot, kvs_paged_decode_scored,
                  kvs_paged_decode_scored_workspace_size, new_pools_fp8, kvs_compact_paged_fp8,
                  kvs_paged_decode_fp8, kvs_copy_blocks_fp8, kvs_prefill_attn_lse_chunk, kvs_window_score_chunk,
                  kvs_gather_paged, kvs_paged_decode_scored_fp8, kvs_probe_stream_read,
                  kvs_probe_timestamp, kvs_paged_decode_scored_select, kvs_paged_decode_scored_select_fp8,
                  kvs_paged_decode_noalloc)
from .allocator import BlockAllocator
from .pipeline import (layer_policy, keep_counts, prefill_compress_layer, prefill_compress_layer_chunked,
                       prefix_rows_reused, prefill_compress_admission)
from .prefix_cache import BlockHashIndex, chained_block_keys

__all__ = [
    "lib", "KvsError", "BLOCK_SIZE", "LIB_PATH",
    "kvs_prefill_attn_lse", "kvs_window_score", "kvs_topk_select", "kvs_compact_paged", "kvs_topk_compact",
    "kvs_paged_decode", "kvs_paged_decode_workspace_size", "kvs_copy_blocks", "new_pools",
    "kvs_slot_init", "kvs_decode_select_slot", "kvs_paged_decode_scored", "kvs_paged_decode_scored_workspace_size",
    "new_pools_fp8", "kvs_compact_paged_fp8", "kvs_paged_decode_fp8", "kvs_copy_blocks_fp8",
    "kvs_prefill_attn_lse_chunk", "kvs_window_score_chunk", "kvs_gather_paged", "kvs_paged_decode_scored_fp8",
    "kvs_probe_stream_read", "kvs_probe_timestamp", "kvs_paged_decode_noalloc",
    "kvs_paged_decode_scored_select", "kvs_paged_decode_scored_select_fp8",
    "BlockAllocator", "layer_policy", "keep_counts", "prefill_compress_layer",
    "prefill_compress_layer_chunked", "prefix_rows_reused", "prefill_compress_admission", "BlockHashIndex",
    "chained_block_keys",
]
