"""Pins for oracle.lifecycle on its own (CPU only): hand-worked admission / decode / finish
traces whose tables, reference counts and free lists were worked out by hand from reading R15,
per-operation invariants on the oracle's own state over the continuous-batch trace, and
planted mistakes that each of these must catch.

Sources: [PAG] "How paging works" (a block is taken when a token's slot opens one),
"Sharing blocks between sequences" (reference counts; a shared block is copied before it is
written), "Related techniques" (a finished sequence returns its blocks at once); [KVS] Key
techniques 1 (first three layers full, later layers a budget).
"""
import collections

import numpy as np
import pytest

import workloads as wl
from oracle.lifecycle import CacheLifecycle
from oracle.paged import RefcountError, NoBlocksError, blocks_for

# Two layers: layer 0 keeps every token, layer 1 keeps k = 32 (two blocks).  Shared prefix
# P = 48 tokens (three blocks).  Twelve blocks per layer, free lists start 0..11.
BUDGETS = [None, 32]
POOL = [12, 12]
P = 48

# sequence -> (group, prompt length); A and B share group 0's prefix (n > 48), C does not.
A, B, C = 0, 1, 2
PROMPTS = {A: (0, 64), B: (0, 50), C: (1, 40)}

OPS = [("admit", A), ("decode", A), ("admit", B), ("admit", C), ("finish", A), ("decode", B),
       ("finish", B), ("finish", C)]


def _state(tables, refs, free):
    return dict(tables=tables, refs=refs, free=free)


# Expected state after each op, worked by hand.  refs lists only the blocks with a non-zero
# count, per layer; tables maps (seq, layer) -> table.
#
# With the prefix carried by the compressed layer too:
#   admit A (n=64, shares): group 0's prefix takes blocks 0,1,2 in layer 0, then 0,1,2 in
#     layer 1 (group reference: count 1).  Layer 0: A adds a reference to 0,1,2 (count 2)
#     and takes 3 for tokens 48..63.  Layer 1: k_eff = 32 -> 2 blocks; A adds a reference to
#     0,1,2, swaps entry 0 (count 2 -> fresh 3, 0 back to 1) and entry 1 (fresh 4), and drops
#     entry 2 (count 1: the group's).
#   decode A: layer 0 slot 64 opens a block (64 % 16 == 0) -> 4; layer 1 slot 32 -> 5.
#   admit B (n=50, shares, group live): layer 0 maps 0,1,2 (count 3) + 5 for tokens 48..49;
#     layer 1 swaps entries 0,1 for 6,7, drops 2.
#   admit C (n=40, no share): layer 0 takes 6,7,8; layer 1 (k_eff 32) takes 8,9.
#   finish A: layer 0: 0,1,2 -> 2, 3 and 4 freed; layer 1: 3,4,5 freed.
#   decode B: layer 0 slot 50 (50 % 16 = 2) takes nothing; layer 1 slot 32 takes 10.
#   finish B (last sharer of group 0): layer 0: 0,1,2 -> 1, 5 freed, then the group's
#     references free 0,1,2; layer 1: 6,7,10 freed, then the group's 0,1,2.
#   finish C: layer 0: 6,7,8; layer 1: 8,9.
EXPECTED_CARRIED = [
    _state({(A, 0): [0, 1, 2, 3], (A, 1): [3, 4]},
           [{0: 2, 1: 2, 2: 2, 3: 1}, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1}],
           [[4, 5, 6, 7, 8, 9, 10, 11], [5, 6, 7, 8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [3, 4, 5]},
           [{0: 2, 1: 2, 2: 2, 3: 1, 4: 1}, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1, 5: 1}],
           [[5, 6, 7, 8, 9, 10, 11], [6, 7, 8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [3, 4, 5], (B, 0): [0, 1, 2, 5], (B, 1): [6, 7]},
           [{0: 3, 1: 3, 2: 3, 3: 1, 4: 1, 5: 1}, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1, 5: 1, 6: 1, 7: 1}],
           [[6, 7, 8, 9, 10, 11], [8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [3, 4, 5], (B, 0): [0, 1, 2, 5], (B, 1): [6, 7],
            (C, 0): [6, 7, 8], (C, 1): [8, 9]},
           [{0: 3, 1: 3, 2: 3, 3: 1, 4: 1, 5: 1, 6: 1, 7: 1, 8: 1},
            {0: 1, 1: 1, 2: 1, 3: 1, 4: 1, 5: 1, 6: 1, 7: 1, 8: 1, 9: 1}],
           [[9, 10, 11], [10, 11]]),
    _state({(B, 0): [0, 1, 2, 5], (B, 1): [6, 7], (C, 0): [6, 7, 8], (C, 1): [8, 9]},
           [{0: 2, 1: 2, 2: 2, 5: 1, 6: 1, 7: 1, 8: 1}, {0: 1, 1: 1, 2: 1, 6: 1, 7: 1, 8: 1, 9: 1}],
           [[9, 10, 11, 3, 4], [10, 11, 3, 4, 5]]),
    _state({(B, 0): [0, 1, 2, 5], (B, 1): [6, 7, 10], (C, 0): [6, 7, 8], (C, 1): [8, 9]},
           [{0: 2, 1: 2, 2: 2, 5: 1, 6: 1, 7: 1, 8: 1}, {0: 1, 1: 1, 2: 1, 6: 1, 7: 1, 8: 1, 9: 1, 10: 1}],
           [[9, 10, 11, 3, 4], [11, 3, 4, 5]]),
    _state({(C, 0): [6, 7, 8], (C, 1): [8, 9]},
           [{6: 1, 7: 1, 8: 1}, {8: 1, 9: 1}],
           [[9, 10, 11, 3, 4, 5, 0, 1, 2], [11, 3, 4, 5, 6, 7, 10, 0, 1, 2]]),
    _state({},
           [{}, {}],
           [[9, 10, 11, 3, 4, 5, 0, 1, 2, 6, 7, 8], [11, 3, 4, 5, 6, 7, 10, 0, 1, 2, 8, 9]]),
]

# With the prefix carried by full layers only: group 0's prefix exists in layer 0 alone, and
# each member of it takes two fresh blocks in layer 1 (the same as C, which shares nothing).
#   admit A: layer 0 as above ([0,1,2] + 3); layer 1 takes 0,1.
#   decode A: layer 0 takes 4; layer 1 slot 32 takes 2.
#   admit B: layer 0 [0,1,2] + 5; layer 1 takes 3,4.
#   admit C: layer 0 takes 6,7,8; layer 1 takes 5,6.
#   finish A: layer 0 frees 3,4 (0,1,2 -> 2); layer 1 frees 0,1,2.
#   decode B: layer 1 slot 32 takes 7.
#   finish B: layer 0 frees 5, then the group's 0,1,2; layer 1 frees 3,4,7.
#   finish C: layer 0 frees 6,7,8; layer 1 frees 5,6.
EXPECTED_FULL_ONLY = [
    _state({(A, 0): [0, 1, 2, 3], (A, 1): [0, 1]},
           [{0: 2, 1: 2, 2: 2, 3: 1}, {0: 1, 1: 1}],
           [[4, 5, 6, 7, 8, 9, 10, 11], [2, 3, 4, 5, 6, 7, 8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [0, 1, 2]},
           [{0: 2, 1: 2, 2: 2, 3: 1, 4: 1}, {0: 1, 1: 1, 2: 1}],
           [[5, 6, 7, 8, 9, 10, 11], [3, 4, 5, 6, 7, 8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [0, 1, 2], (B, 0): [0, 1, 2, 5], (B, 1): [3, 4]},
           [{0: 3, 1: 3, 2: 3, 3: 1, 4: 1, 5: 1}, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1}],
           [[6, 7, 8, 9, 10, 11], [5, 6, 7, 8, 9, 10, 11]]),
    _state({(A, 0): [0, 1, 2, 3, 4], (A, 1): [0, 1, 2], (B, 0): [0, 1, 2, 5], (B, 1): [3, 4],
            (C, 0): [6, 7, 8], (C, 1): [5, 6]},
           [{0: 3, 1: 3, 2: 3, 3: 1, 4: 1, 5: 1, 6: 1, 7: 1, 8: 1}, {0: 1, 1: 1, 2: 1, 3: 1, 4: 1, 5: 1, 6: 1}],
           [[9, 10, 11], [7, 8, 9, 10, 11]]),
    _state({(B, 0): [0, 1, 2, 5], (B, 1): [3, 4], (C, 0): [6, 7, 8], (C, 1): [5, 6]},
           [{0: 2, 1: 2, 2: 2, 5: 1, 6: 1, 7: 1, 8: 1}, {3: 1, 4: 1, 5: 1, 6: 1}],
           [[9, 10, 11, 3, 4], [7, 8, 9, 10, 11, 0, 1, 2]]),
    _state({(B, 0): [0, 1, 2, 5], (B, 1): [3, 4, 7], (C, 0): [6, 7, 8], (C, 1): [5, 6]},
           [{0: 2, 1: 2, 2: 2, 5: 1, 6: 1, 7: 1, 8: 1}, {3: 1, 4: 1, 5: 1, 6: 1, 7: 1}],
           [[9, 10, 11, 3, 4], [8, 9, 10, 11, 0, 1, 2]]),
    _state({(C, 0): [6, 7, 8], (C, 1): [5, 6]},
           [{6: 1, 7: 1, 8: 1}, {5: 1, 6: 1}],
           [[9, 10, 11, 3, 4, 5, 0, 1, 2], [8, 9, 10, 11, 0, 1, 2, 3, 4, 7]]),
    _state({},
           [{}, {}],
           [[9, 10, 11, 3, 4, 5, 0, 1, 2, 6, 7, 8], [8, 9, 10, 11, 0, 1, 2, 3, 4, 7, 5, 6]]),
]


def _apply(lc, op, seq):
    if op == "admit":
        g, n = PROMPTS[seq]
        lc.admit(seq, g, n)
    elif op == "decode":
        for l in range(len(lc.budgets)):
            lc.decode_one(seq, l)
    else:
        lc.finish(seq)


def run_worked_trace(cls, carried):
    lc = cls(BUDGETS, POOL, P, prefix_in_compressed=carried)
    expected = EXPECTED_CARRIED if carried else EXPECTED_FULL_ONLY
    for (op, seq), want in zip(OPS, expected):
        _apply(lc, op, seq)
        assert lc.table == want["tables"], f"tables after {op} {seq}"
        for l in range(2):
            refs = {b: c for b, c in enumerate(lc.alloc[l].ref) if c}
            assert refs == want["refs"][l], f"reference counts of layer {l} after {op} {seq}"
            assert list(lc.alloc[l].free) == want["free"][l], f"free list of layer {l} after {op} {seq}"


@pytest.mark.parametrize("carried", [True, False])
def test_hand_worked_trace(carried):
    run_worked_trace(CacheLifecycle, carried)


def test_worked_trace_allocator_calls():
    """The first admission's calls, in order, as R15 fixes them (prefix of every layer first)."""
    lc = CacheLifecycle(BUDGETS, POOL, P)
    lc.admit(A, 0, 64)
    assert lc.ops == [("alloc", 0, 0), ("alloc", 0, 1), ("alloc", 0, 2), ("alloc", 1, 0), ("alloc", 1, 1),
                      ("alloc", 1, 2), ("incref", 0, 0), ("incref", 0, 1), ("incref", 0, 2), ("alloc", 0, 3),
                      ("incref", 1, 0), ("incref", 1, 1), ("incref", 1, 2), ("cow", 1, 0, 3, True),
                      ("cow", 1, 1, 4, True), ("decref", 1, 2)]


# ---------------------------------------------------------------- invariants on the oracle's state
def check_state(lc):
    """What R15 and the allocator's rules fix about any reachable state, from public state only."""
    P16 = lc.P // 16
    by_layer = collections.defaultdict(list)
    for (s, l), t in lc.table.items():
        by_layer[l].append((s, t))
    pre_by_layer = collections.defaultdict(list)
    for (l, g), pre in lc.prefix.items():
        pre_by_layer[l].append(pre)
        assert len(pre) == P16
    for l, alloc in enumerate(lc.alloc):
        ref = np.asarray(alloc.ref)
        for s, t in by_layer[l]:
            assert len(t) == blocks_for(lc.tokens[(s, l)]), "a table holds exactly ceil(tokens/16) blocks"
            if lc.budgets[l] is not None:
                # compressed tables are private: a copy-on-write result is never shared
                assert np.all(ref[t] == 1), "a compressed layer's block is shared"
            g = lc.shares_in[s]
            if g is not None and lc.budgets[l] is None:
                assert t[:P16] == lc.prefix[(l, g)], "a full layer maps its group's prefix first"
        # every reference is held by a table or a group prefix, and by nothing else
        held = [b for _, t in by_layer[l] for b in t] + [b for pre in pre_by_layer[l] for b in pre]
        holders = np.bincount(np.asarray(held, dtype=np.int64), minlength=alloc.num_blocks)
        assert np.array_equal(holders, ref), f"counts differ from holders, layer {l}"
        free = np.asarray(list(alloc.free), dtype=np.int64)
        assert len(np.unique(free)) == len(free), "a block is free twice"
        assert np.array_equal(np.sort(free), np.flatnonzero(ref == 0)), \
            "live and free blocks do not partition the pool"
    # a group's prefix exists exactly while it has a live sharing member, in the layers that carry it
    live_groups = {g for s, g in lc.shares_in.items() if g is not None}
    for l in range(len(lc.budgets)):
        carried = {g for (layer, g) in lc.prefix if layer == l}
        assert carried == (live_groups if lc.carries_prefix(l) else set())


def finish_checked(lc, seq):
    """finish() frees exactly the sequence's private blocks, plus its group's prefix if it was the
    last sharer, appended to the free lists in release order."""
    g = lc.shares_in[seq]
    last = g is not None and sum(1 for x in lc.shares_in.values() if x == g) == 1
    before = [list(a.free) for a in lc.alloc]
    expect = []
    for l, alloc in enumerate(lc.alloc):
        own = [b for b in lc.table[(seq, l)] if alloc.ref[b] == 1]
        pre = [b for b in lc.prefix.get((l, g), [])] if last else []
        # a prefix block is freed with the last sharer: the group's reference plus, in full
        # layers, that sharer's own
        pre = [b for b in pre if alloc.ref[b] == (2 if lc.budgets[l] is None else 1)]
        expect.append(own + pre)
    lc.finish(seq)
    for l, alloc in enumerate(lc.alloc):
        after = list(alloc.free)
        assert after[:len(before[l])] == before[l]
        assert after[len(before[l]):] == expect[l], f"finish of {seq} frees the wrong blocks in layer {l}"


def drive_checked(cls, carried, iterations, every=1):
    w = wl.WORKLOADS[5]
    sizes = wl.mix_pool_sizes(w)
    lc = cls(w.budgets, sizes, w.prefix_len, prefix_in_compressed=carried)
    live = []
    for it, (admitted, finished) in enumerate(wl.mix_trace(w, iterations)):
        for sq in admitted:
            lc.admit(sq.seq_id, sq.group, sq.n)
            live.append(sq.seq_id)
            if it % every == 0:
                check_state(lc)
        for sid in sorted(live):
            for l in range(w.n_layers):
                lc.decode_one(sid, l)
        if it % every == 0:
            check_state(lc)
        for sid in finished:
            finish_checked(lc, sid)
            live.remove(sid)
            if it % every == 0:
                check_state(lc)
    return lc, live


@pytest.mark.parametrize("carried", [True, False])
def test_invariants_over_the_mix(carried):
    lc, live = drive_checked(CacheLifecycle, carried, 420, every=20)
    w = wl.WORKLOADS[5]
    # compressed layers hold the live sequences' caches and, with the policy, one prefix per live group
    for l, k in enumerate(w.budgets):
        if k is None:
            continue
        taken = lc.alloc[l].num_blocks - lc.alloc[l].num_free()
        caches = sum(blocks_for(lc.tokens[(s, l)]) for s in live)
        groups = len({lc.shares_in[s] for s in live} - {None})
        assert taken == caches + (groups * (w.prefix_len // 16) if carried else 0)
    for sid in list(live):
        finish_checked(lc, sid)
    check_state(lc)
    for l, a in enumerate(lc.alloc):
        assert a.num_free() == a.num_blocks


def test_exhaustion_and_misuse_raise():
    lc = CacheLifecycle([None], [4], 0)
    lc.admit(0, 0, 64)                       # four blocks: the pool is full
    with pytest.raises(NoBlocksError):
        lc.decode_one(0, 0)                  # slot 64 opens a fifth block
    lc2 = CacheLifecycle([None], [8], 0)
    lc2.admit(0, 0, 20)
    lc2.finish(0)
    with pytest.raises(KeyError):
        lc2.finish(0)


# ---------------------------------------------------------------- planted mistakes
class CowAllPrefixEntries(CacheLifecycle):
    """Mistake: a compressed layer swaps every prefix entry, not only those the compaction writes."""

    def admit(self, seq, group, n):
        shared_before = {key: list(v) for key, v in self.prefix.items()}
        super().admit(seq, group, n)
        for l, k in enumerate(self.budgets):
            if k is not None and self.shares_in[seq] is not None and (l, group) in self.prefix:
                t = self.table[(seq, l)]
                need = blocks_for(self.tokens[(seq, l)])
                pre = shared_before.get((l, group), self.prefix[(l, group)])
                for e in range(need, len(pre)):
                    # the entry was released by the correct rule; the mistake swaps it instead
                    self._ref(l, pre[e])
                    t.append(self._write_shared(l, pre[e]))


class NoGroupReference(CacheLifecycle):
    """Mistake: the group holds no reference of its own; the first member's is the allocation."""

    def _ref(self, l, b):
        if self.alloc[l].ref[b] == 1 and self._fresh.get((l, b)):
            self._fresh[(l, b)] = False          # the creating member takes over the allocation
            return
        super()._ref(l, b)

    def _take(self, l):
        b = super()._take(l)
        self._fresh[(l, b)] = self._creating
        return b

    def admit(self, seq, group, n):
        self._creating = self.P > 0 and n > self.P and not self.members.get(group)
        super().admit(seq, group, n)
        self._creating = False

    def finish(self, seq):
        g = self.shares_in.get(seq)
        if g is not None and len(self.members.get(g, ())) == 1:
            # no group reference to drop
            for l in range(len(self.budgets)):
                self.prefix.pop((l, g), None)
        super().finish(seq)

    def __init__(self, *a, **k):
        self._fresh, self._creating = {}, False
        super().__init__(*a, **k)


class DecodeSlotOffByOne(CacheLifecycle):
    """Mistake: the block is opened when L % 16 == 0 (L = length after the token), not (L-1)."""

    def decode_one(self, seq, l):
        L = self.tokens[(seq, l)] + 1
        if L % 16 == 0:
            self.table[(seq, l)].append(self._take(l))
        self.tokens[(seq, l)] = L


@pytest.mark.parametrize("mutant", [CowAllPrefixEntries, NoGroupReference, DecodeSlotOffByOne])
@pytest.mark.parametrize("carried", [True, False])
def test_planted_mistakes_fail_a_pin(mutant, carried):
    caught = []
    for pin in (lambda: run_worked_trace(mutant, carried), lambda: drive_checked(mutant, carried, 40)):
        try:
            pin()
        except (AssertionError, RefcountError, NoBlocksError, KeyError):
            caught.append(True)
        else:
            caught.append(False)
    if mutant is CowAllPrefixEntries and not carried:
        # without a prefix in compressed layers there is nothing to swap: the mistake cannot occur
        assert not any(caught)
    else:
        assert any(caught), f"{mutant.__name__} passed every pin"
