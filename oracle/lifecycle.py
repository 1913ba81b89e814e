"""Paged-cache lifecycle under continuous batching with shared prefixes (oracle; test infrastructure).

Sources: [PAG] "How paging works" (take a block only when the last one is full), "Sharing
blocks between sequences" (reference counts; a shared block is copied before it is written),
"Related techniques" (a finished sequence returns its blocks at once); [KVS] Key techniques 1
(per-layer block tables; first three layers full, later layers a budget k_l).

Reading R15 (what the pages leave open), applied per layer with one allocator per layer:
  * a prompt of n > P tokens (P = shared prefix length, whole blocks) shares its group's P/16
    prefix blocks; the group itself holds one reference to them while it has a live sharing
    member, and each sharing member holds one more;
  * full layer: the member maps the prefix blocks and takes fresh blocks for tokens P..n-1;
  * compressed layer: the member maps the prefix blocks, then every table entry the
    compaction writes (the first ceil(k_eff/16)) is replaced copy-on-write and its
    references to the other prefix entries are dropped;
  * non-sharing prompts take ceil(k_eff/16) fresh blocks;
  * a decoded token takes a fresh block when its slot opens one;
  * a finished sequence drops every block it maps, and the group drops its prefix
    references when its last sharing member finishes.
Admissions run layer 0 first; the group's prefix blocks for all layers are taken before the
first member maps any of them.  Every allocator call is logged as
(op, layer, block[, new_block, copied]).
"""
from __future__ import annotations

from .paged import BlockAllocator, blocks_for


class CacheLifecycle:
    def __init__(self, budgets, num_blocks, prefix_len):
        self.budgets = list(budgets)
        self.P = prefix_len
        self.alloc = [BlockAllocator(nb) for nb in num_blocks]
        self.prefix = {}          # (layer, group) -> list of blocks
        self.live_sharers = {}    # group -> count
        self.table = {}           # (seq, layer) -> list of blocks
        self.tokens = {}          # (seq, layer) -> cached tokens
        self.shares_in = {}       # seq -> group or None
        self.ops = []

    def _new(self, l):
        b = self.alloc[l].alloc()
        self.ops.append(("alloc", l, b))
        return b

    def _inc(self, l, b):
        self.alloc[l].incref(b)
        self.ops.append(("incref", l, b))

    def _dec(self, l, b):
        self.alloc[l].decref(b)
        self.ops.append(("decref", l, b))

    def _copy_on_write(self, l, b):
        nb, copied = self.alloc[l].cow(b)
        self.ops.append(("cow", l, b, nb, copied))
        return nb

    def admit(self, seq, group, n):
        layers = range(len(self.budgets))
        sharing = self.P > 0 and n > self.P
        self.shares_in[seq] = group if sharing else None
        if sharing:
            if self.live_sharers.get(group, 0) == 0:
                for l in layers:
                    self.prefix[(l, group)] = [self._new(l) for _ in range(self.P // 16)]
            self.live_sharers[group] = self.live_sharers.get(group, 0) + 1
        for l in layers:
            k = self.budgets[l]
            k_eff = n if k is None or k >= n else k
            if not sharing:
                blocks = [self._new(l) for _ in range(blocks_for(k_eff))]
            else:
                pre = self.prefix[(l, group)]
                for b in pre:
                    self._inc(l, b)
                if k is None:
                    blocks = list(pre) + [self._new(l) for _ in range(blocks_for(n) - len(pre))]
                else:
                    need = blocks_for(k_eff)
                    blocks = []
                    for t, b in enumerate(pre):
                        if t < need:
                            blocks.append(self._copy_on_write(l, b))
                        else:
                            self._dec(l, b)
                    while len(blocks) < need:
                        blocks.append(self._new(l))
            self.table[(seq, l)] = blocks
            self.tokens[(seq, l)] = k_eff

    def decode_one(self, seq, l):
        L = self.tokens[(seq, l)] + 1
        if (L - 1) % 16 == 0:
            self.table[(seq, l)].append(self._new(l))
        self.tokens[(seq, l)] = L

    def finish(self, seq):
        for l in range(len(self.budgets)):
            for b in self.table.pop((seq, l)):
                self._dec(l, b)
            self.tokens.pop((seq, l))
        group = self.shares_in.pop(seq)
        if group is not None:
            self.live_sharers[group] -= 1
            if self.live_sharers[group] == 0:
                for l in range(len(self.budgets)):
                    for b in self.prefix.pop((l, group)):
                        self._dec(l, b)
