"""Prompt prefix reuse by hashes of full blocks (host side).

[PAG] Ultralytics glossary, "PagedAttention", "Sharing blocks between sequences": block
sharing extends to different requests by hashing full blocks, which is how vLLM caches
prompts.  [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM",
Conclusion: chunked prefill and prefix caching are listed there as not yet supported.

A block's key is a digest of its 16 token ids chained with the key of the block before it,
so a block can only match together with the whole prefix in front of it.  A new prompt
reuses the longest run of leading full blocks whose keys are known, but always leaves its
last min(alpha, n) tokens (at least one) to compute: those query rows produce the step's
output and the window score.  The reused rows' K/V come back from the cache
(``kvs_gather_paged``) and only the remaining rows are prefilled as a chunk
(``kvs_prefill_attn_lse_chunk``).
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Sequence, Tuple

import numpy as np

from ._lib import BLOCK_SIZE


def chained_block_keys(tokens: Sequence[int], block: int = BLOCK_SIZE) -> List[bytes]:
    """One key per full block: blake2b(previous key || the block's token ids as int64)."""
    ids = np.ascontiguousarray(np.asarray(tokens, dtype=np.int64))
    keys: List[bytes] = []
    prev = b""
    for start in range(0, len(ids) - block + 1, block):
        h = hashlib.blake2b(prev, digest_size=32)
        h.update(ids[start:start + block].tobytes())
        prev = h.digest()
        keys.append(prev)
    return keys


class BlockHashIndex:
    """Known block keys, each with the (sequence, table entry) whose block holds it."""

    def __init__(self, block: int = BLOCK_SIZE):
        self.block = block
        self._owner: Dict[bytes, Tuple[int, int]] = {}
        self._by_seq: Dict[int, List[bytes]] = {}

    def register(self, seq: int, tokens: Sequence[int]) -> int:
        """Make the full blocks of a cached prompt findable; returns how many were new."""
        added = 0
        for i, key in enumerate(chained_block_keys(tokens, self.block)):
            if key not in self._owner:
                self._owner[key] = (seq, i)
                self._by_seq.setdefault(seq, []).append(key)
                added += 1
        return added

    def forget(self, seq: int) -> None:
        """The sequence's blocks are gone (it finished): drop the keys it provided."""
        for key in self._by_seq.pop(seq, []):
            self._owner.pop(key, None)

    def match(self, tokens: Sequence[int], alpha: int) -> Tuple[int, List[Tuple[int, int]]]:
        """(tokens that can be reused, the (sequence, table entry) of each reused block)."""
        n = len(tokens)
        must_compute = max(min(alpha, n), 1)
        reusable_blocks = max(n - must_compute, 0) // self.block
        found: List[Tuple[int, int]] = []
        for key in chained_block_keys(tokens[:reusable_blocks * self.block], self.block):
            owner = self._owner.get(key)
            if owner is None:
                break
            found.append(owner)
        return len(found) * self.block, found
