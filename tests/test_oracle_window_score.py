"""Pins for oracle.window_score: closed form at Q = 0, conservation, a second route
through a library softmax, the GQA group sum and the visited-pair count (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import window_score, window_score_from_probs, visited_pairs


def _rand(n, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, hq, d)), r.standard_normal((n, hkv, d))


def _t(x):
    return torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]


def _lib_lse(q, k):
    """LSE [Hq][n] from torch's CPU flash attention (independent of the oracle)."""
    G = q.shape[1] // k.shape[1]
    kk = _t(k).repeat_interleave(G, 1)
    out = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(_t(q), kk, kk, 0.0, True)
    return out[1][0].numpy()


def _lib_probs(q, k):
    """A [Hq][n][n] from torch's attention with V = identity."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    eye = np.tile(np.eye(n)[:, None, :], (1, hkv, 1))
    vt = torch.from_numpy(np.ascontiguousarray(eye.transpose(1, 0, 2)))[None]
    A = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), vt, is_causal=True, enable_gqa=True,
                                                         scale=1 / math.sqrt(d))
    return A[0].numpy()


@pytest.mark.parametrize("n,alpha,G", [(40, 8, 2), (17, 17, 1), (10, 16, 4), (64, 1, 2)])
def test_zero_query_closed_form(n, alpha, G):
    hkv, d = 2, 8
    _, k = _rand(n, G * hkv, hkv, d, 1)
    q = np.zeros((n, G * hkv, d))
    lse = np.tile(np.log(np.arange(1, n + 1)), (G * hkv, 1))      # LSE_j = ln(j+1) at Q = 0
    S = window_score(q, k, lse, alpha)
    a = min(alpha, n)
    ref = np.array([G * sum(1.0 / (j + 1) for j in range(max(i, n - a), n)) for i in range(n)])
    for g in range(hkv):
        np.testing.assert_allclose(S[g], ref, rtol=1e-13, atol=0)


@pytest.mark.parametrize("n,alpha", [(50, 8), (33, 32), (12, 40)])
def test_conservation(n, alpha):
    """Every window row's probabilities sum to one, so the total score of a KV head is G * alpha."""
    hq, hkv, d = 4, 2, 16
    q, k = _rand(n, hq, hkv, d, n)
    S = window_score(q, k, _lib_lse(q, k), alpha)
    np.testing.assert_allclose(S.sum(axis=1), 2 * min(alpha, n), rtol=1e-12)
    assert np.all(S >= 0)


@pytest.mark.parametrize("n,alpha,hq,hkv", [(40, 8, 4, 2), (31, 5, 6, 3), (25, 25, 2, 2)])
def test_two_routes_agree(n, alpha, hq, hkv):
    """Explicit exp(s - LSE) sum == column sums of a library softmax matrix over the window rows."""
    d = 32
    q, k = _rand(n, hq, hkv, d, 100 + n)
    S1 = window_score(q, k, _lib_lse(q, k), alpha)
    S2 = window_score_from_probs(_lib_probs(q, k), alpha, hkv)
    np.testing.assert_allclose(S1, S2, rtol=1e-12, atol=1e-15)


def test_gqa_group_sum():
    """S of a KV head equals the sum of its G query heads scored one by one (Hkv = Hq copies)."""
    n, hq, hkv, d, alpha = 30, 4, 2, 8, 6
    q, k = _rand(n, hq, hkv, d, 7)
    lse = _lib_lse(q, k)
    S = window_score(q, k, lse, alpha)
    k_rep = np.repeat(k, 2, axis=1)                  # query head h paired with its own copy of KV head h // 2
    S_each = window_score(q, k_rep, lse, alpha)
    np.testing.assert_allclose(S, S_each.reshape(hkv, 2, n).sum(1), rtol=1e-13)


def test_window_tokens_only_see_later_rows():
    """Token i inside the window gets rows j >= i only: the score of the last token is the sum of its own
    diagonal probabilities."""
    n, hq, hkv, d, alpha = 20, 2, 1, 8, 5
    q, k = _rand(n, hq, hkv, d, 8)
    A = _lib_probs(q, k)
    S = window_score(q, k, _lib_lse(q, k), alpha)
    assert abs(S[0, n - 1] - (A[0, n - 1, n - 1] + A[1, n - 1, n - 1])) < 1e-13


def test_visited_pairs_counts_the_pages_example():
    """With a 5000-token prompt and a 256-row window only about 5000 x 256 pairs are visited, not 5000 x 5000."""
    v = visited_pairs(5000, 256)
    assert v == sum(range(5000 - 256 + 1, 5001))
    assert v <= 5000 * 256 and v > 0.95 * 5000 * 256
    assert visited_pairs(10, 3) == 8 + 9 + 10
    assert visited_pairs(4, 10) == 1 + 2 + 3 + 4


def test_row_subset_interfaces_equal_full_calls():
    """q_holds_rows / window_only only change what the caller passes, not the result."""
    from oracle import causal_attention
    n, hq, hkv, d = 200, 4, 2, 16
    q, k = _rand(n, hq, hkv, d, 21)
    v = np.random.default_rng(22).standard_normal((n, hkv, d))
    rows = [0, 7, 150, 199]
    O1, l1, m1, e1 = causal_attention(q, k, v, rows=rows)
    O2, l2, m2, e2 = causal_attention(q[rows], k, v, rows=rows, q_holds_rows=True)
    assert np.array_equal(O1, O2) and np.array_equal(l1, l2) and np.array_equal(m1, m2) and np.array_equal(e1, e2)
    lse = causal_attention(q, k, v)[1]
    for alpha in (1, 8, 500):
        a = min(alpha, n)
        S1 = window_score(q, k, lse, alpha)
        S2 = window_score(q[n - a:], k, lse[:, n - a:], alpha, window_only=True)
        assert np.array_equal(S1, S2)
