"""Pins of the chunked-prefill reading (R25) and the block-hash prefix match (R26)."""
import numpy as np
import pytest

import oracle
from oracle import prefix


def _rand(rng, n, hq, hkv, d):
    return (rng.standard_normal((n, hq, d)), rng.standard_normal((n, hkv, d)), rng.standard_normal((n, hkv, d)))


@pytest.mark.parametrize("c0,c1", [(0, 37), (37, 80), (64, 128), (127, 128)])
def test_chunk_rows_equal_full_prefill_rows(c0, c1):
    """A chunk attending keys [0, c1) gives the one-pass prefill's rows (no carry needed)."""
    rng = np.random.default_rng(c0 + 7 * c1)
    q, k, v = _rand(rng, 128, 4, 2, 16)
    O, lse, m, l = oracle.causal_attention(q, k, v)
    Oc, lc, mc, llc = oracle.causal_attention(q[c0:c1], k[:c1], v[:c1], rows=range(c0, c1), q_holds_rows=True)
    np.testing.assert_allclose(Oc, O[c0:c1], rtol=1e-12, atol=1e-12)
    np.testing.assert_allclose(lc, lse[:, c0:c1], rtol=1e-12, atol=1e-12)


def test_chunked_window_score_equals_full():
    """The window score from the last chunk's rows and LSE equals the one from the whole prompt."""
    rng = np.random.default_rng(5)
    n, alpha = 90, 16
    q, k, v = _rand(rng, n, 4, 2, 16)
    _, lse, _, _ = oracle.causal_attention(q, k, v)
    S = oracle.window_score(q, k, lse, alpha)
    c0 = 60                                               # last chunk rows [60, 90) hold the window
    _, lc, _, _ = oracle.causal_attention(q[c0:], k, v, rows=range(c0, n), q_holds_rows=True)
    a = min(alpha, n)
    Sc = oracle.window_score(q[n - a:], k, lc[:, n - a - c0:], alpha, window_only=True)
    np.testing.assert_allclose(Sc, S, rtol=1e-12, atol=1e-14)


def _common_blocks(a, b, block=16):
    """Brute force: leading full blocks on which two token sequences agree."""
    m = 0
    while (m + 1) * block <= min(len(a), len(b)) and np.array_equal(a[m * block:(m + 1) * block],
                                                                    b[m * block:(m + 1) * block]):
        m += 1
    return m


def test_match_is_the_longest_common_block_prefix():
    rng = np.random.default_rng(11)
    base = rng.integers(0, 32000, 300)
    seqs = {}
    idx = prefix.PrefixIndex()
    for sid in range(6):
        cut = int(rng.integers(0, 300))
        t = np.concatenate([base[:cut], rng.integers(0, 32000, int(rng.integers(0, 200)))])
        seqs[sid] = t
        idx.register(sid, t)
    for trial in range(40):
        cut = int(rng.integers(0, 300))
        new = np.concatenate([base[:cut], rng.integers(0, 32000, int(rng.integers(1, 150)))])
        alpha = int(rng.integers(1, 40))
        got, src = idx.match(new, alpha)
        limit = (len(new) - max(min(alpha, len(new)), 1)) // 16
        want = min(limit, max(_common_blocks(new, t) for t in seqs.values()))
        assert got == 16 * want
        for i, (sid, bi) in enumerate(src):   # each reused block really holds the same tokens
            assert bi == i and np.array_equal(seqs[sid][16 * i:16 * i + 16], new[16 * i:16 * i + 16])


def test_a_block_matches_only_with_its_prefix():
    """Equal block contents after different prefixes hash differently (chaining)."""
    blk = np.arange(16)
    a = np.concatenate([np.zeros(16, np.int64), blk])
    b = np.concatenate([np.ones(16, np.int64), blk])
    ha, hb = prefix.block_hashes(a), prefix.block_hashes(b)
    assert ha[1] != hb[1] and ha[0] != hb[0]
    assert prefix.block_hashes(a)[1] == prefix.block_hashes(np.concatenate([a, [5, 6]]))[1]
    assert len(prefix.block_hashes(np.arange(31))) == 1          # a partial block has no hash


def test_match_leaves_the_window_to_compute():
    idx = prefix.PrefixIndex()
    t = np.arange(64)
    idx.register(0, t)
    assert idx.match(t, alpha=1)[0] == 48           # a fully cached prompt still computes its last block
    assert idx.match(t, alpha=20)[0] == 32          # 44 tokens may be cached: 2 whole blocks
    assert idx.match(t[:16], alpha=1)[0] == 0
    idx.remove(0)
    assert idx.match(t, alpha=1)[0] == 0
