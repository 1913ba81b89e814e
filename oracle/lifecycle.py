"""Paged-cache lifecycle under continuous batching with shared prefixes (oracle; TEST INFRASTRUCTURE).

Only the tests may use this module; the product never imports it.

Sources: [PAG] "How paging works" (a request takes a block only when its last one is full,
from anywhere in the pool), "Sharing blocks between sequences" (several sequences map one
physical block, each block counts its users, a shared block is copied before it is written),
"Related techniques" (continuous batching: a finished sequence returns its blocks at once);
[KVS] Key techniques 1 (every layer has its own block table; the first three layers keep
every token, later layers a budget k_l).

Reading R15 (the pages leave the policy open).  One allocator per layer.  A prompt of n
tokens shares its group's prefix of P tokens (whole blocks) when n > P.  A group's prefix
exists while the group has at least one live sharing member; the group itself holds one
reference to each prefix block, every sharing member one more.  Which layers carry a
shared prefix is a policy:

  * full layers always do: the member maps the P/16 prefix blocks and takes fresh blocks
    for its tokens P..n-1 (the prefix ends on a block boundary, so no shared block is
    written);
  * compressed layers do only under `prefix_in_compressed` (the prefix is then a prompt
    cache that later members read their first P keys and values from).  The member maps
    the prefix, and since the compaction rewrites slots 0..k_eff-1, each of the first
    ceil(k_eff/16) entries it writes is replaced copy-on-write (no data copy: every live
    slot is overwritten) and its references to the other prefix entries are dropped.
    Without the policy the member simply takes ceil(k_eff/16) fresh blocks, as a prompt
    that shares nothing does in every compressed layer.

A decoded token is written to slot L-1 of its (sequence, layer), L the length after it;
that slot opens a block when (L-1) is a multiple of 16.  A finished sequence drops every
reference it holds; when a group's last sharing member finishes, the group drops its own.

Order of allocator calls (it fixes the block ids): an admission that creates a group's
prefix first takes the prefix blocks of every carrying layer, layer 0 first; then, layer by
layer, the member's references, copy-on-write swaps (entry order), releases and fresh
blocks.  Every call is logged as (op, layer, block[, new_block, swapped]).
"""
from __future__ import annotations

from .paged import BlockAllocator, blocks_for


class CacheLifecycle:
    def __init__(self, budgets, num_blocks, prefix_len, prefix_in_compressed=True):
        if prefix_len % 16:
            raise ValueError("the shared prefix must be whole blocks")
        self.budgets = list(budgets)
        self.P = prefix_len
        self.prefix_in_compressed = prefix_in_compressed
        self.alloc = [BlockAllocator(nb) for nb in num_blocks]
        self.prefix = {}          # (layer, group) -> the group's prefix blocks in that layer
        self.members = {}         # group -> live sharing members (a set of seq ids)
        self.table = {}           # (seq, layer) -> block table
        self.tokens = {}          # (seq, layer) -> cached tokens
        self.shares_in = {}       # seq -> the group whose prefix it maps, or None
        self.ops = []

    # allocator calls, logged in the order they are made
    def _take(self, l):
        b = self.alloc[l].alloc()
        self.ops.append(("alloc", l, b))
        return b

    def _ref(self, l, b):
        self.alloc[l].incref(b)
        self.ops.append(("incref", l, b))

    def _release(self, l, b):
        self.alloc[l].decref(b)
        self.ops.append(("decref", l, b))

    def _write_shared(self, l, b):
        nb, swapped = self.alloc[l].cow(b)
        self.ops.append(("cow", l, b, nb, swapped))
        return nb

    def carries_prefix(self, l):
        """Whether layer l keeps a group's shared prefix (full layers always; compressed by policy)."""
        return self.budgets[l] is None or self.prefix_in_compressed

    def kept(self, l, n):
        k = self.budgets[l]
        return n if k is None or k >= n else k

    def admit(self, seq, group, n):
        sharing = self.P > 0 and n > self.P
        self.shares_in[seq] = group if sharing else None
        if sharing:
            if not self.members.get(group):
                for l in range(len(self.budgets)):
                    if self.carries_prefix(l):
                        self.prefix[(l, group)] = [self._take(l) for _ in range(self.P // 16)]
            self.members.setdefault(group, set()).add(seq)
        for l in range(len(self.budgets)):
            k_eff = self.kept(l, n)
            need = blocks_for(k_eff)
            if not sharing or not self.carries_prefix(l):
                table = [self._take(l) for _ in range(need)]
            else:
                shared = self.prefix[(l, group)]
                for b in shared:
                    self._ref(l, b)
                if self.budgets[l] is None:
                    # the suffix P..n-1 starts on a block boundary: the prefix stays shared
                    table = shared + [self._take(l) for _ in range(need - len(shared))]
                else:
                    # compaction rewrites slots 0..k_eff-1: swap the entries it writes, drop the rest
                    table = []
                    for e, b in enumerate(shared):
                        if e < need:
                            table.append(self._write_shared(l, b))
                        else:
                            self._release(l, b)
                    table += [self._take(l) for _ in range(need - len(table))]
            self.table[(seq, l)] = table
            self.tokens[(seq, l)] = k_eff

    def decode_one(self, seq, l):
        slot = self.tokens[(seq, l)]          # the new token's slot, L - 1
        if slot % 16 == 0:
            self.table[(seq, l)].append(self._take(l))
        self.tokens[(seq, l)] = slot + 1

    def finish(self, seq):
        for l in range(len(self.budgets)):
            for b in self.table.pop((seq, l)):
                self._release(l, b)
            del self.tokens[(seq, l)]
        group = self.shares_in.pop(seq)
        if group is not None:
            self.members[group].discard(seq)
            if not self.members[group]:
                del self.members[group]
                for l in range(len(self.budgets)):
                    for b in self.prefix.pop((l, group), []):
                        self._release(l, b)
