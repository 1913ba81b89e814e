"""Host bookkeeping of a paged, per-layer KV cache under continuous batching.

[PAG] Ultralytics glossary, "PagedAttention": "How paging works" (a request takes a new
block only when its last one is full, from any free block), "Sharing blocks between
sequences" (several sequences map one physical block, a reference count per block, copy
before writing a shared block), "Related techniques" (continuous batching: a finished
sequence's blocks go back to the free pool at once).  [KVS] Novita AI, "How KV Sparsity
Achieves 1.5x Acceleration for vLLM", Key techniques 1: each layer has its own block-table
strategy; the first three layers keep every token, the later ones a budget k_l.

Every layer has its own pool and its own native allocator (kvs_alloc_*).  The manager only
decides which blocks each (sequence, layer) maps; the caller launches the kernels that fill
them (kvs_compact_paged for prompts and shared prefixes, kvs_paged_decode for appends).

Prefix sharing.  Sequences of one group share a prefix of `prefix_len` tokens (whole blocks)
when their prompt is longer than it.  While any such member is live the group holds one
reference to the prefix blocks of every layer that carries them; each member adds its own:
  * full layers always carry the prefix: the member keeps the shared blocks and writes only
    its suffix, from slot prefix_len on (a block boundary, so no shared block is written);
  * compressed layers carry it only with `prefix_in_compressed` (the prefix is then a prompt
    cache: a later member reads its first prefix_len keys and values back from those blocks
    instead of recomputing them).  The compaction overwrites slots 0..k_eff-1, so the member
    takes copy-on-write replacements for those ceil(k_eff/16) table entries (no data copy:
    every live slot is overwritten) and drops its references to the remaining prefix entries.
    Without it a compressed layer holds nothing of the prefix: each member takes
    ceil(k_eff/16) fresh blocks, so the layer holds only the compressed caches.
When the group's last sharing member finishes, the group's references go too.
"""
from __future__ import annotations

from typing import Dict, List, Optional, Sequence, Tuple

from ._lib import BLOCK_SIZE
from .allocator import BlockAllocator


def _blocks(tokens: int) -> int:
    return -(-tokens // BLOCK_SIZE)


class LayerPlan:
    __slots__ = ("layer", "table", "kept", "dst_offset", "new_prefix")

    def __init__(self, layer, table, kept, dst_offset, new_prefix):
        self.layer = layer
        self.table = table              # block ids of this (sequence, layer)
        self.kept = kept                # tokens the compaction writes (k_eff, or the suffix length)
        self.dst_offset = dst_offset    # slot of the first written token
        self.new_prefix = new_prefix    # the group's prefix blocks were just created: write them


class PagedKVCache:
    def __init__(self, budgets: Sequence[Optional[int]], num_blocks: Sequence[int], prefix_len: int = 0,
                 record: bool = False, prefix_in_compressed: bool = True):
        if prefix_len % BLOCK_SIZE:
            raise ValueError("the shared prefix must be whole blocks")
        self.budgets = list(budgets)
        self.n_layers = len(self.budgets)
        self.alloc = [BlockAllocator(nb) for nb in num_blocks]
        self.prefix_len = prefix_len
        self.prefix_in_compressed = prefix_in_compressed
        self.prefix_blocks: List[Dict[int, List[int]]] = [dict() for _ in range(self.n_layers)]
        self.sharers: Dict[int, int] = {}                      # group -> live sharing members
        self.tables: Dict[Tuple[int, int], List[int]] = {}     # (seq, layer) -> block ids
        self.length: Dict[Tuple[int, int], int] = {}           # (seq, layer) -> cached tokens
        self.group_of: Dict[int, Optional[int]] = {}           # seq -> group it shares with (or None)
        self.log: Optional[list] = [] if record else None

    # --- allocator calls, recorded -------------------------------------------------------
    def _rec(self, *op):
        if self.log is not None:
            self.log.append(op)

    def _alloc(self, l):
        b = self.alloc[l].alloc()
        self._rec("alloc", l, b)
        return b

    def _incref(self, l, b):
        self.alloc[l].incref(b)
        self._rec("incref", l, b)

    def _decref(self, l, b):
        self.alloc[l].decref(b)
        self._rec("decref", l, b)

    def _cow(self, l, b):
        nb, copied = self.alloc[l].cow(b)
        self._rec("cow", l, b, nb, copied)
        return nb

    # --- lifecycle -----------------------------------------------------------------------
    def carries_prefix(self, layer: int) -> bool:
        """Whether the layer keeps a group's shared prefix (full layers always; compressed by policy)."""
        return self.budgets[layer] is None or self.prefix_in_compressed

    def kept_tokens(self, layer: int, n: int) -> int:
        k = self.budgets[layer]
        return n if (k is None or k >= n) else k

    def admit(self, seq: int, group: int, n: int) -> List[LayerPlan]:
        """Map the blocks of a new prompt of n tokens in every layer."""
        P = self.prefix_len // BLOCK_SIZE
        shares = self.prefix_len > 0 and n > self.prefix_len
        new_prefix = False
        if shares:
            if self.sharers.get(group, 0) == 0:                 # the group's prefix is created now
                for l in range(self.n_layers):
                    if self.carries_prefix(l):
                        self.prefix_blocks[l][group] = [self._alloc(l) for _ in range(P)]
                new_prefix = True
            self.sharers[group] = self.sharers.get(group, 0) + 1
        self.group_of[seq] = group if shares else None
        plans = []
        for l in range(self.n_layers):
            kept = self.kept_tokens(l, n)
            if shares and self.carries_prefix(l):
                table = list(self.prefix_blocks[l][group])
                for b in table:
                    self._incref(l, b)
                if self.budgets[l] is None:                      # full layer: keep the prefix shared
                    table += [self._alloc(l) for _ in range(_blocks(n) - P)]
                    plans.append(LayerPlan(l, table, n - self.prefix_len, self.prefix_len, new_prefix))
                else:                                            # compressed: COW what compaction writes
                    c = _blocks(kept)
                    for t in range(min(c, P)):
                        table[t] = self._cow(l, table[t])
                    for t in range(c, P):
                        self._decref(l, table[t])
                    table = table[:c] + [self._alloc(l) for _ in range(c - P)]
                    plans.append(LayerPlan(l, table, kept, 0, new_prefix))
            else:
                table = [self._alloc(l) for _ in range(_blocks(kept))]
                plans.append(LayerPlan(l, table, kept, 0, False))
            self.tables[(seq, l)] = table
            self.length[(seq, l)] = kept
        return plans

    def append(self, seq: int, layer: int) -> List[int]:
        """Reserve the slot of one decoded token; a block is taken when that slot opens one."""
        key = (seq, layer)
        L = self.length[key] + 1
        if (L - 1) % BLOCK_SIZE == 0:
            self.tables[key].append(self._alloc(layer))
        self.length[key] = L
        return self.tables[key]

    def finish(self, seq: int) -> None:
        """Return every block the sequence maps (shared ones lose one reference)."""
        for l in range(self.n_layers):
            for b in self.tables.pop((seq, l)):
                self._decref(l, b)
            del self.length[(seq, l)]
        group = self.group_of.pop(seq)
        if group is not None:
            self.sharers[group] -= 1
            if self.sharers[group] == 0:                        # last sharer: drop the group's references
                for l in range(self.n_layers):
                    for b in self.prefix_blocks[l].pop(group, []):
                        self._decref(l, b)

    def slot_usage(self, layer: int) -> Tuple[int, int]:
        """(slots holding a live token, slots in blocks taken from the pool) for one layer.

        [PAG] "How paging works": paging wastes only the unfilled tail of each sequence's last
        block.  A shared prefix block counts once, however many tables map it.
        """
        used = sum(self.prefix_len for _ in self.prefix_blocks[layer])
        for (sid, l), n in self.length.items():
            if l == layer:
                # a sharing member's full-layer table maps the prefix blocks counted above
                shared = self.group_of.get(sid) is not None and self.budgets[layer] is None
                used += n - (self.prefix_len if shared else 0)
        taken = self.alloc[layer].num_blocks - self.alloc[layer].num_free()
        return used, taken * BLOCK_SIZE

    def num_free(self, layer: int) -> int:
        return self.alloc[layer].num_free()

    def free_list(self, layer: int) -> List[int]:
        return self.alloc[layer].free_list()
