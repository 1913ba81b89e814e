"""Pins for oracle.decode: the last prefill row (a different code path), a library
attention call, the Q = 0 closed form and order invariance (CPU only)."""
import math

import numpy as np
import torch

from oracle import causal_attention, decode_attention, select_keep, BlockAllocator, blocks_for
from oracle import compact_into_pool, gather_rows


def _rand(n, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, hq, d)), r.standard_normal((n, hkv, d)), r.standard_normal((n, hkv, d))


def test_equals_last_prefill_row():
    n, hq, hkv, d = 45, 8, 2, 16
    q, k, v = _rand(n, hq, hkv, d, 1)
    O, lse, _, _ = causal_attention(q, k, v)
    o, l = decode_attention(q[n - 1], k, v)
    np.testing.assert_allclose(o, O[n - 1], rtol=0, atol=1e-13)
    np.testing.assert_allclose(l, lse[:, n - 1], rtol=0, atol=1e-13)


def test_matches_library_attention():
    L, hq, hkv, d = 70, 8, 2, 32
    _, k, v = _rand(L, hq, hkv, d, 2)
    q = np.random.default_rng(3).standard_normal((hq, d))
    o, _ = decode_attention(q, k, v)
    t = lambda x: torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(torch.from_numpy(q)[None, :, None, :], t(k), t(v),
                                                           enable_gqa=True)
    np.testing.assert_allclose(o, ref[0, :, 0].numpy(), rtol=0, atol=1e-13)


def test_zero_query_is_mean_of_values():
    L, hq, hkv, d = 19, 4, 2, 8
    _, k, v = _rand(L, hq, hkv, d, 4)
    o, lse = decode_attention(np.zeros((hq, d)), k, v)
    for h in range(hq):
        np.testing.assert_allclose(o[h], v[:, h // 2].mean(0), rtol=0, atol=1e-14)
    np.testing.assert_allclose(lse, math.log(L), rtol=0, atol=1e-14)


def test_order_invariance():
    L, hq, hkv, d = 33, 4, 1, 8
    _, k, v = _rand(L, hq, hkv, d, 5)
    q = np.random.default_rng(6).standard_normal((hq, d))
    p = np.random.default_rng(7).permutation(L)
    o1, l1 = decode_attention(q, k, v)
    o2, l2 = decode_attention(q, k[p], v[p])
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-13)
    np.testing.assert_allclose(l1, l2, rtol=0, atol=1e-13)


def test_budget_at_least_n_is_full_cache_through_the_table():
    """With k >= n the 'compressed' cache is the full cache: decode through the table equals the plain one."""
    n, hq, hkv, d, alpha = 40, 4, 2, 8, 8
    q, k, v = _rand(n, hq, hkv, d, 8)
    keep = np.stack([select_keep(np.zeros(n), n, alpha, 64) for _ in range(hkv)])
    a = BlockAllocator(8, initial_free_order=[5, 1, 7, 0, 2, 3, 4, 6])
    table = [a.alloc() for _ in range(blocks_for(n))]
    pk = np.zeros((8, hkv, 16, d)); pv = np.zeros_like(pk)
    compact_into_pool(k, v, keep, table, pk, pv)
    o1, _ = decode_attention(q[-1], gather_rows(pk, table, n), gather_rows(pv, table, n))
    o2, _ = decode_attention(q[-1], k, v)
    np.testing.assert_allclose(o1, o2, rtol=0, atol=1e-14)
