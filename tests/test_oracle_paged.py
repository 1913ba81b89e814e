"""Pins for oracle.paged: the PagedAttention page's worked example (golden fixture),
block-table round trips, allocator order and refcount invariants, copy-on-write (CPU only)."""
import json
import os

import numpy as np
import pytest

from oracle import BlockAllocator, blocks_for, write_rows, gather_rows, compact_into_pool
from oracle.paged import NoBlocksError, RefcountError

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "paged_worked_example.json")


def test_worked_example_from_the_page():
    g = json.load(open(GOLDEN))
    bs, d = g["block_size"], g["head_dim"]
    assert bs == 16
    alloc = BlockAllocator(g["pool_blocks"], initial_free_order=g["free_blocks"])
    n = g["num_tokens"]
    table = [alloc.alloc() for _ in range(blocks_for(n))]
    assert table == g["expected_block_table"]
    pool = np.zeros((g["pool_blocks"], 1, bs, d))
    keys = np.random.default_rng(0).standard_normal((n, 1, d))
    write_rows(pool, table, keys)
    intact = np.array_equal(gather_rows(pool, table, n), keys)
    assert intact == g["expected_keys_intact"]
    assert len(table) * bs - n == g["expected_unused_slots_paged"]
    assert g["reservation_tokens"] - n == g["expected_unused_slots_reserved"]
    assert list(alloc.free) == [2, 33]
    assert alloc.ref[0] == 1 and alloc.ref[41] == 1 and alloc.ref[2] == 0   # unlisted blocks are in use


@pytest.mark.parametrize("n,off", [(1, 0), (16, 0), (17, 0), (40, 0), (33, 5), (64, 16), (100, 31)])
def test_round_trip_with_offset(n, off):
    r = np.random.default_rng(n + off)
    hkv, d = 3, 8
    pool = np.full((50, hkv, 16, d), np.nan)
    table = list(r.permutation(50)[: blocks_for(n + off)])
    rows = r.standard_normal((n, hkv, d))
    write_rows(pool, table, rows, off=off)
    back = gather_rows(pool, table, n + off)
    np.testing.assert_array_equal(back[off:], rows)
    assert np.all(np.isnan(back[:off]))                    # slots before the offset untouched


def test_compaction_per_head_keep():
    r = np.random.default_rng(3)
    n, hkv, d, k = 70, 2, 4, 20
    K = r.standard_normal((n, hkv, d))
    V = r.standard_normal((n, hkv, d))
    keep = np.stack([np.sort(r.choice(n, k, replace=False)) for _ in range(hkv)])
    pk = np.zeros((10, hkv, 16, d)); pv = np.zeros_like(pk)
    table = [9, 2, 4]
    compact_into_pool(K, V, keep, table, pk, pv)
    gk, gv = gather_rows(pk, table, k), gather_rows(pv, table, k)
    for h in range(hkv):
        np.testing.assert_array_equal(gk[:, h], K[keep[h], h])
        np.testing.assert_array_equal(gv[:, h], V[keep[h], h])
    # keep-all writes the source unchanged
    pk2 = np.zeros((10, hkv, 16, d)); pv2 = np.zeros_like(pk2)
    tab = list(range(blocks_for(n)))
    compact_into_pool(K, V, None, tab, pk2, pv2)
    np.testing.assert_array_equal(gather_rows(pk2, tab, n), K)


def test_blocks_for():
    assert [blocks_for(x) for x in (0, 1, 15, 16, 17, 32, 33, 400, 4000)] == [0, 1, 1, 1, 2, 2, 3, 25, 250]


def test_fifo_order_and_exhaustion():
    a = BlockAllocator(4)
    assert [a.alloc() for _ in range(4)] == [0, 1, 2, 3]
    with pytest.raises(NoBlocksError):
        a.alloc()
    a.decref(2); a.decref(0)
    assert [a.alloc(), a.alloc()] == [2, 0]


def test_refcount_misuse():
    a = BlockAllocator(3)
    b = a.alloc()
    a.decref(b)
    with pytest.raises(RefcountError):
        a.decref(b)
    with pytest.raises(RefcountError):
        a.incref(b)


def test_copy_on_write():
    a = BlockAllocator(6)
    b = a.alloc()
    a.incref(b); a.incref(b)              # three sharers
    nb, copied = a.cow(b)
    assert copied and nb != b and a.ref[b] == 2 and a.ref[nb] == 1
    nb2, copied2 = a.cow(nb)               # private block: written in place
    assert not copied2 and nb2 == nb
    a.decref(b); a.decref(b)
    assert b in a.free


@pytest.mark.parametrize("seed", range(10))
def test_random_ops_invariants(seed):
    """Live and free blocks partition the pool; counts never go negative; the free list is FIFO."""
    r = np.random.default_rng(seed)
    N = 32
    a = BlockAllocator(N, initial_free_order=r.permutation(N))
    live = {}
    expected_free = list(a.free)
    for _ in range(600):
        op = r.integers(0, 4)
        if op == 0:
            if expected_free:
                b = a.alloc()
                assert b == expected_free.pop(0)
                live[b] = 1
            else:
                with pytest.raises(NoBlocksError):
                    a.alloc()
        elif op == 1 and live:
            b = list(live)[r.integers(len(live))]
            a.incref(b); live[b] += 1
        elif op == 2 and live:
            b = list(live)[r.integers(len(live))]
            a.decref(b); live[b] -= 1
            if live[b] == 0:
                del live[b]; expected_free.append(b)
        elif op == 3 and live:
            b = list(live)[r.integers(len(live))]
            if live[b] > 1 and not expected_free:
                with pytest.raises(NoBlocksError):
                    a.cow(b)
                continue
            nb, copied = a.cow(b)
            if live[b] > 1:
                assert copied and nb == expected_free.pop(0)
                live[b] -= 1; live[nb] = 1
            else:
                assert not copied and nb == b
        assert list(a.free) == expected_free
        assert set(a.free).isdisjoint(live)
        assert len(a.free) + len(live) == N
        assert all(a.ref[b] == c for b, c in live.items())
