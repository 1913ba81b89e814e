"""Pins of the decode-time scoring / eviction oracle (R20, R21) against closed forms,
invariants, a hand-worked case and the plain decode oracle."""
import math

import numpy as np
import pytest

import oracle


def _cache(rng, hkv, cap, n, d, positions=None):
    k = rng.standard_normal((hkv, cap, d))
    v = rng.standard_normal((hkv, cap, d))
    score = rng.random((hkv, cap))
    pos = np.full((hkv, cap), -1, dtype=np.int64)
    for g in range(hkv):
        pos[g, :n] = positions[g] if positions is not None else np.arange(n)
    return oracle.SlotCache(k, v, score, pos, n, cap)


def test_select_slot_worked_example():
    # four slots, alpha 1, the new token at position 4: position 3 is protected; among
    # positions 0..2 the lowest score (1.0, slot 1) goes
    score = np.array([3.0, 1.0, 2.0, 0.5])
    pos = np.array([0, 1, 2, 3])
    assert oracle.select_slot(score, pos, 4, 4, 4, 1) == 1
    # alpha 2 protects positions 2 and 3 as well: still slot 1
    assert oracle.select_slot(score, pos, 4, 4, 4, 2) == 1
    # equal lowest scores: the older position goes
    score = np.array([2.0, 1.0, 1.0, 0.5])
    pos = np.array([7, 5, 2, 9])
    assert oracle.select_slot(score, pos, 4, 4, 10, 1) == 2
    # room left: append at the first free slot, whatever the scores
    assert oracle.select_slot(score, pos, 3, 4, 10, 1) == 3
    with pytest.raises(ValueError):
        oracle.select_slot(score, np.array([7, 8, 9, 6]), 4, 4, 10, 4)


def test_select_slot_brute_force():
    rng = np.random.default_rng(3)
    for _ in range(300):
        cap = int(rng.integers(2, 9))
        alpha = int(rng.integers(1, cap))
        new_pos = int(rng.integers(cap, 3 * cap))
        pos = rng.choice(new_pos, size=cap, replace=False)
        score = rng.integers(0, 4, size=cap).astype(float)      # many ties
        eligible = [t for t in range(cap) if pos[t] < new_pos - alpha]
        if not eligible:
            continue
        t = oracle.select_slot(score, pos, cap, cap, new_pos, alpha)
        assert t in eligible
        assert all((score[t], pos[t]) <= (score[u], pos[u]) for u in eligible)


def test_no_eviction_matches_plain_decode():
    """With room in the cache the step is the plain decode over the appended tokens."""
    rng = np.random.default_rng(5)
    hq, hkv, d, n, cap = 8, 2, 16, 11, 40
    c = _cache(rng, hkv, cap, n, d)
    for step in range(5):
        q = rng.standard_normal((hq, d))
        nk, nv = rng.standard_normal((hkv, d)), rng.standard_normal((hkv, d))
        n0 = c.n
        o, lse, dst = oracle.decode_step(c, q, nk, nv, 100 + step, 4)
        assert list(dst) == [n0] * hkv
        k_ctx = np.transpose(c.k[:, :c.n], (1, 0, 2))
        v_ctx = np.transpose(c.v[:, :c.n], (1, 0, 2))
        o_ref, lse_ref = oracle.decode_attention(q, k_ctx, v_ctx)
        np.testing.assert_allclose(o, o_ref, rtol=0, atol=1e-12)
        np.testing.assert_allclose(lse, lse_ref, rtol=0, atol=1e-12)


def test_scores_gain_G_per_step_and_uniform_at_zero_query():
    rng = np.random.default_rng(7)
    hq, hkv, d, cap = 12, 3, 8, 9
    c = _cache(rng, hkv, cap, cap, d)
    G = hq // hkv
    for step in range(6):
        before = c.score.copy()
        q = rng.standard_normal((hq, d)) if step % 2 else np.zeros((hq, d))
        o, lse, dst = oracle.decode_step(c, q, rng.standard_normal((hkv, d)), rng.standard_normal((hkv, d)),
                                         50 + step, 2)
        gain = c.score.copy()
        for g in range(hkv):
            before[g, dst[g]] = 0.0                # the new token started at 0
        np.testing.assert_allclose((gain - before).sum(axis=1), G, rtol=0, atol=1e-12)
        if step % 2 == 0:                          # q = 0: every live slot gains G / n
            np.testing.assert_allclose(gain - before, G / cap, rtol=0, atol=1e-12)
            np.testing.assert_allclose(lse, math.log(cap), rtol=0, atol=1e-12)


def test_eviction_invariants_over_many_steps():
    rng = np.random.default_rng(11)
    hq, hkv, d, alpha, cap, n = 8, 4, 16, 3, 12, 30
    k_rows = rng.standard_normal((n, hkv, d))
    v_rows = rng.standard_normal((n, hkv, d))
    S = rng.random((hkv, n))
    keep = np.stack([np.sort(np.concatenate([rng.choice(n - alpha, cap - alpha, replace=False),
                                             np.arange(n - alpha, n)])) for _ in range(hkv)])
    c = oracle.init_cache(k_rows, v_rows, S, keep, cap)
    for g in range(hkv):
        np.testing.assert_array_equal(c.score[g], S[g, keep[g]])
        np.testing.assert_array_equal(c.k[g], k_rows[keep[g], g])
    dsts = []
    for step in range(40):
        new_pos = n + step
        o, lse, dst = oracle.decode_step(c, rng.standard_normal((hq, d)), rng.standard_normal((hkv, d)),
                                         rng.standard_normal((hkv, d)), new_pos, alpha)
        dsts.append(dst)
        assert c.n == cap
        for g in range(hkv):
            assert len(set(c.pos[g])) == cap                     # no token twice
            assert set(range(new_pos - alpha + 1, new_pos + 1)) <= set(c.pos[g])   # recent tokens stay
    # heads choose their victims independently
    assert any(len(set(d_)) > 1 for d_ in dsts)
