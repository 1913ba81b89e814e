"""CPU oracle for the KV-sparsity prefill-and-compress path (TEST INFRASTRUCTURE).

This package is test infrastructure.  Only the tests, the smoke check in
``__graft_entry__`` and the ``cpu_baseline`` leg of ``bench.py`` may import it.
The product path (the HIP library and its Python binding) never imports,
calls or links anything here, and this package imports nothing from it.

Everything is plain numpy in float64, written from the two source pages:

  [KVS]  Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM"
         (blog post; the Arabic and Japanese editions carry the same text).
  [PAG]  Ultralytics glossary, "PagedAttention".

Modules and the step each one follows:

  attention     causal softmax attention with the per-row max and sum
                ([KVS] Key techniques 2, "Attention modification": the
                attention formula and the FlashAttention2 figure, first Fig. 7)
  window_score  the observation-window score S ([KVS] same section, the
                PyramidKV-style score and the modified-FlashAttention figure,
                second Fig. 7)
  topk          per-layer, per-KV-head selection of the tokens to keep
                ([KVS] same section; System model for "high score and near")
  paged         block allocator, block tables, compaction into 16-token
                blocks, copy-on-write ([PAG] "How paging works", "Sharing
                blocks between sequences", "Related techniques")
  decode        attention of one new token over a paged cache ([PAG] "How
                paging works"; [KVS] Key techniques 2, last paragraph)
  eviction      decode-time scores and the replacement of the lowest-score
                token in a full compressed layer ([KVS] Key techniques 1, step
                preparation; Key techniques 2, last paragraph)
  fp8           the 8-bit (E4M3) cache: encoding, per-row scales, the
                quantized compaction and decode append ([PAG] "Related
                techniques")
  prefix        chunked prefill and the block-hash prefix match ([PAG]
                "Sharing blocks between sequences"; [KVS] Conclusion)

Readings taken where the pages are silent or garbled are named R1..R26 in the
docstrings; each one is listed with its justification in the design notes.
Every function is pinned by the CPU tests (``pytest -m "not gpu"``); none is
"parity unpinned".
"""
from .attention import causal_attention, attention_probs
from .window_score import window_score, window_score_from_probs, visited_pairs
from .topk import select_keep, keep_count
from .paged import BlockAllocator, blocks_for, write_rows, gather_rows, compact_into_pool
from .decode import decode_attention
from .eviction import SlotCache, init_cache, select_slot, decode_step
from . import fp8
from . import prefix

__all__ = [
    "causal_attention", "attention_probs",
    "window_score", "window_score_from_probs", "visited_pairs",
    "select_keep", "keep_count",
    "BlockAllocator", "blocks_for", "write_rows", "gather_rows", "compact_into_pool",
    "decode_attention",
    "SlotCache", "init_cache", "select_slot", "decode_step",
    "fp8", "prefix",
]
