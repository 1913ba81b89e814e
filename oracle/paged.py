"""Paged KV storage: block allocator, block tables, compaction (oracle; test infrastructure).

Source: [PAG] "How paging works": the cache is split into blocks of a fixed
number of tokens (16 by default in vLLM) that may sit anywhere in GPU memory; a
request gets a new block only when its last one is full, taken from wherever a
free block is; a per-request block table records the order, and the attention
kernel follows the table block by block.  The page's worked example pops the
free blocks from the front of a list and writes token pos to block
table[pos // 16], slot pos % 16.  [PAG] "Sharing blocks between sequences":
several sequences may map the same physical block, each block carries a
reference count, and a sequence that must write a block still used by others
copies it first (copy-on-write).  [PAG] "Related techniques", continuous
batching: a finished sequence's blocks go back to the free pool at once.
[KVS] Key techniques 1: the first three layers keep a full cache, the later
ones a reduced one, each with its own block table.

Readings:
  R12 pool layout (logical) [num_blocks][Hkv][16][d]; one table per
      (sequence, layer) shared by all KV heads, since every head keeps the same
      number of tokens.
  R13 the free list is first-in first-out: allocation pops the front, a block
      whose count drops to zero is appended at the back; the initial order is
      0..N-1 unless given.
  R15 copy-on-write: a block with count > 1 is replaced by a fresh block and
      the old one loses a reference; the caller copies the data only when a
      live slot of the old block will not be overwritten.
"""
from __future__ import annotations

import collections
from typing import Iterable, List, Optional, Sequence

import numpy as np

BLOCK = 16


class NoBlocksError(RuntimeError):
    pass


class RefcountError(RuntimeError):
    pass


class BlockAllocator:
    """FIFO free list plus a reference count per block (R13, R15)."""

    def __init__(self, num_blocks: int, initial_free_order: Optional[Iterable[int]] = None):
        if num_blocks <= 0:
            raise ValueError("num_blocks must be positive")
        self.num_blocks = num_blocks
        order = list(range(num_blocks)) if initial_free_order is None else [int(b) for b in initial_free_order]
        if len(set(order)) != len(order) or any(b < 0 or b >= num_blocks for b in order):
            raise ValueError("initial free order must be distinct ids in [0, num_blocks)")
        self.free = collections.deque(order)
        # Blocks missing from the initial free list belong to other requests (the page's
        # example has a 64-block pool with five free blocks): they start with count 1.
        listed = set(order)
        self.ref = [0 if b in listed else 1 for b in range(num_blocks)]
        self.log: List[tuple] = []

    def _valid(self, b: int):
        if not (0 <= b < self.num_blocks):
            raise ValueError(f"block {b} out of range")

    def alloc(self) -> int:
        if not self.free:
            self.log.append(("alloc", -1))
            raise NoBlocksError("pool exhausted")
        b = self.free.popleft()
        self.ref[b] = 1
        self.log.append(("alloc", b))
        return b

    def incref(self, b: int) -> int:
        self._valid(b)
        if self.ref[b] == 0:
            raise RefcountError(f"incref of free block {b}")
        self.ref[b] += 1
        self.log.append(("incref", b))
        return self.ref[b]

    def decref(self, b: int) -> int:
        self._valid(b)
        if self.ref[b] == 0:
            raise RefcountError(f"decref of free block {b}")
        self.ref[b] -= 1
        if self.ref[b] == 0:
            self.free.append(b)
        self.log.append(("decref", b))
        return self.ref[b]

    def cow(self, b: int):
        """Return (block to write, copied?): a shared block is swapped for a fresh one."""
        self._valid(b)
        if self.ref[b] == 0:
            raise RefcountError(f"cow of free block {b}")
        if self.ref[b] == 1:
            self.log.append(("cow", b, b))
            return b, False
        nb = self.alloc()
        self.decref(b)
        self.log.append(("cow", b, nb))
        return nb, True

    def num_free(self) -> int:
        return len(self.free)


def blocks_for(num_tokens: int, block_size: int = BLOCK) -> int:
    """ceil(num_tokens / block_size): blocks a request of that length occupies."""
    return -(-num_tokens // block_size)


def write_rows(pool: np.ndarray, table: Sequence[int], rows: np.ndarray, off: int = 0) -> None:
    """pool[table[p // 16], :, p % 16, :] = rows[t] for p = off + t (pool [blocks][Hkv][16][d], rows [t][Hkv][d])."""
    for t in range(rows.shape[0]):
        p = off + t
        pool[table[p // BLOCK], :, p % BLOCK, :] = rows[t]


def gather_rows(pool: np.ndarray, table: Sequence[int], length: int) -> np.ndarray:
    """Read a sequence back through its table: [length][Hkv][d] (the page's pool[table] gather)."""
    blocks = pool[np.asarray(table[:blocks_for(length)], dtype=np.int64)]     # [nb][Hkv][16][d]
    nb, hkv, bs, d = blocks.shape
    return blocks.transpose(0, 2, 1, 3).reshape(nb * bs, hkv, d)[:length]


def compact_into_pool(k: np.ndarray, v: np.ndarray, keep: Optional[np.ndarray], table: Sequence[int],
                      pool_k: np.ndarray, pool_v: np.ndarray, off: int = 0) -> None:
    """Write the kept rows of every KV head, in kept order, to slots off.. of the table.

    keep is [Hkv][k_eff] (per-head token indices) or None to keep every row.
    """
    n, hkv, d = k.shape
    if keep is None:
        keep = np.tile(np.arange(n), (hkv, 1))
    for h in range(hkv):
        for t, i in enumerate(keep[h]):
            p = off + t
            pool_k[table[p // BLOCK], h, p % BLOCK, :] = k[i, h, :]
            pool_v[table[p // BLOCK], h, p % BLOCK, :] = v[i, h, :]
