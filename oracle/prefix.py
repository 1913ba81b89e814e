"""Chunked prefill and prefix caching by block hashes (oracle; test infrastructure).

Source: [PAG] Ultralytics glossary, "PagedAttention", "Sharing blocks between sequences": the
sharing of physical blocks extends to different requests by hashing full blocks, which is how
vLLM caches prompts.  [KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM",
Conclusion: chunked prefill and prefix caching are listed as not yet supported there.

Readings:
  R25 a prompt may be prefilled in chunks of query rows: rows [c0, c1) attend keys [0, c1)
      with the causal rule of the full prompt (row i sees keys <= i).  Every row sees all of
      its keys inside its own chunk, so its O and LSE are those of the one-pass prefill and
      no statistic is carried between chunks; the window score needs the LSE of the last
      min(alpha, n) rows, which the chunk holding them provides.
  R26 a block's hash covers the block's tokens and the hash of the block before it, so a
      block matches only together with everything before it; a new prompt reuses the
      longest run of leading full blocks whose hashes are registered, but always leaves its
      last min(alpha, n) tokens (at least one) to compute, since their query rows give the
      output and the window score.

The attention of a chunk is the pinned causal-attention oracle asked for the chunk's rows
(``attention.causal_attention(..., rows=..., q_holds_rows=True)``); this module adds the hash
chain and the match rule.
"""
from __future__ import annotations

import hashlib
from typing import Dict, List, Sequence, Tuple

import numpy as np

from .paged import BLOCK


def block_hashes(tokens: Sequence[int], block: int = BLOCK) -> List[bytes]:
    """Chained hashes of the full blocks of a token sequence (a partial last block has none)."""
    t = np.asarray(tokens, dtype=np.int64)
    out: List[bytes] = []
    prev = b""
    for b in range(len(t) // block):
        h = hashlib.sha256(prev + t[b * block:(b + 1) * block].tobytes()).digest()
        out.append(h)
        prev = h
    return out


class PrefixIndex:
    """Registered block hashes, each with the (sequence, block index) that first wrote it."""

    def __init__(self, block: int = BLOCK):
        self.block = block
        self.where: Dict[bytes, Tuple[int, int]] = {}

    def register(self, seq: int, tokens: Sequence[int]) -> None:
        for i, h in enumerate(block_hashes(tokens, self.block)):
            self.where.setdefault(h, (seq, i))

    def remove(self, seq: int) -> None:
        self.where = {h: v for h, v in self.where.items() if v[0] != seq}

    def match(self, tokens: Sequence[int], alpha: int) -> Tuple[int, List[Tuple[int, int]]]:
        """(cached tokens, the (sequence, block) each reused block comes from), per R26."""
        n = len(tokens)
        keep_rows = max(min(alpha, n), 1)
        limit = (n - keep_rows) // self.block        # most blocks that may be reused
        found: List[Tuple[int, int]] = []
        for h in block_hashes(tokens, self.block)[:limit]:
            if h not in self.where:
                break
            found.append(self.where[h])
        return len(found) * self.block, found
