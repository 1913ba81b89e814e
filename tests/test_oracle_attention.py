"""Pins for oracle.attention: an independent library implementation, closed forms,
invariants, brute force and structural properties (CPU only)."""
import math

import numpy as np
import pytest
import torch

from oracle import causal_attention, attention_probs

pytestmark = pytest.mark.filterwarnings("ignore::UserWarning")


def _rand(n, hq, hkv, d, seed):
    r = np.random.default_rng(seed)
    return r.standard_normal((n, hq, d)), r.standard_normal((n, hkv, d)), r.standard_normal((n, hkv, d))


def _t(x):  # [n][H][d] -> [1][H][n][d]
    return torch.from_numpy(np.ascontiguousarray(x.transpose(1, 0, 2)))[None]


@pytest.mark.parametrize("n,hq,hkv,d", [(1, 2, 1, 8), (37, 4, 2, 16), (130, 8, 2, 64), (65, 4, 4, 32)])
def test_matches_torch_cpu_flash_attention(n, hq, hkv, d):
    """torch's CPU flash attention (an online-softmax implementation) in fp64 returns O and the LSE."""
    q, k, v = _rand(n, hq, hkv, d, n + d)
    O, lse, m, l = causal_attention(q, k, v)
    G = hq // hkv
    ref_o = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), _t(v), is_causal=True, enable_gqa=True)
    out, ref_lse = torch.ops.aten._scaled_dot_product_flash_attention_for_cpu(
        _t(q), _t(k).repeat_interleave(G, 1), _t(v).repeat_interleave(G, 1), 0.0, True)[:2]
    np.testing.assert_allclose(O, ref_o[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(O, out[0].numpy().transpose(1, 0, 2), rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse[0].numpy(), rtol=0, atol=1e-12)


def test_invariants_rows_sum_to_one_and_lse_split():
    n, hq, hkv, d = 50, 4, 2, 16
    q, k, v = _rand(n, hq, hkv, d, 3)
    A = attention_probs(q, k)
    np.testing.assert_allclose(A.sum(-1), 1.0, rtol=0, atol=1e-13)
    assert np.all(A[:, np.triu_indices(n, 1)[0], np.triu_indices(n, 1)[1]] == 0)
    O, lse, m, l = causal_attention(q, k, v)
    np.testing.assert_allclose(lse, m + np.log(l), rtol=0, atol=1e-13)
    # m is the row maximum of the scaled logits: exp(s - m) peaks at exactly 1, so 1 <= l <= j + 1
    assert np.all(l >= 1.0 - 1e-12) and np.all(l <= np.arange(1, n + 1)[None, :] + 1e-9)
    # O is A V for each head's group
    G = hq // hkv
    for h in range(hq):
        np.testing.assert_allclose(O[:, h], A[h] @ v[:, h // G], rtol=0, atol=1e-12)


def test_zero_query_closed_form():
    n, hq, hkv, d = 40, 4, 2, 8
    _, k, v = _rand(n, hq, hkv, d, 5)
    q = np.zeros((n, hq, d))
    O, lse, m, l = causal_attention(q, k, v)
    j = np.arange(n)
    np.testing.assert_allclose(lse, np.log(j + 1)[None, :].repeat(hq, 0), rtol=0, atol=1e-13)
    A = attention_probs(q, k)
    np.testing.assert_allclose(A[0, 7, :8], 1 / 8, rtol=0, atol=1e-15)
    cummean = np.cumsum(v, axis=0) / (j + 1)[:, None, None]
    for h in range(hq):
        np.testing.assert_allclose(O[:, h], cummean[:, h // 2], rtol=0, atol=1e-12)


def test_single_token():
    q, k, v = _rand(1, 4, 2, 16, 9)
    O, lse, m, l = causal_attention(q, k, v)
    for h in range(4):
        np.testing.assert_allclose(O[0, h], v[0, h // 2], rtol=0, atol=1e-15)
        assert abs(lse[h, 0] - q[0, h] @ k[0, h // 2] / 4.0) < 1e-14


def test_key_shift_invariance():
    """Adding c to every key adds q_j.c to row j's logits: O is unchanged and LSE moves by scale*q_j.c."""
    n, hq, hkv, d = 33, 4, 2, 16
    q, k, v = _rand(n, hq, hkv, d, 11)
    c = np.random.default_rng(1).standard_normal(d)
    O1, lse1, _, _ = causal_attention(q, k, v)
    O2, lse2, _, _ = causal_attention(q, k + c, v)
    np.testing.assert_allclose(O1, O2, rtol=0, atol=1e-11)
    np.testing.assert_allclose(lse2 - lse1, (q @ c).T / 4.0, rtol=0, atol=1e-11)


def test_causality():
    n, hq, hkv, d = 30, 2, 1, 8
    q, k, v = _rand(n, hq, hkv, d, 12)
    O1, lse1, _, _ = causal_attention(q, k, v)
    k2, v2 = k.copy(), v.copy()
    k2[20:] += 5.0
    v2[20:] -= 3.0
    O2, lse2, _, _ = causal_attention(q, k2, v2)
    np.testing.assert_array_equal(O1[:20], O2[:20])
    np.testing.assert_array_equal(lse1[:, :20], lse2[:, :20])
    assert np.abs(O1[20:] - O2[20:]).max() > 1e-3


def test_brute_force_scalar_loops():
    """Pure-Python scalar loops (math.exp, no numpy matmul) on tiny inputs."""
    n, hq, hkv, d = 5, 4, 2, 3
    q, k, v = _rand(n, hq, hkv, d, 13)
    O, lse, _, _ = causal_attention(q, k, v)
    sc = 1 / math.sqrt(d)
    for h in range(hq):
        g = h // 2
        for j in range(n):
            logits = [sc * sum(q[j, h, c] * k[i, g, c] for c in range(d)) for i in range(j + 1)]
            tot = sum(math.exp(x) for x in logits)
            assert abs(lse[h, j] - math.log(tot)) < 1e-12
            for c in range(d):
                ref = sum(math.exp(logits[i]) / tot * v[i, g, c] for i in range(j + 1))
                assert abs(O[j, h, c] - ref) < 1e-12


def test_row_subset_and_chunking():
    n, hq, hkv, d = 300, 4, 2, 16
    q, k, v = _rand(n, hq, hkv, d, 14)
    O, lse, m, l = causal_attention(q, k, v, row_chunk=64)
    O2, lse2, _, _ = causal_attention(q, k, v, row_chunk=4096)
    np.testing.assert_allclose(O, O2, rtol=0, atol=1e-13)
    rows = [0, 63, 64, 150, 299]
    O3, lse3, _, _ = causal_attention(q, k, v, rows=rows, row_chunk=2)
    np.testing.assert_allclose(O3, O[rows], rtol=0, atol=1e-13)
    np.testing.assert_allclose(lse3, lse[:, rows], rtol=0, atol=1e-13)


def test_gqa_grouping():
    """Changing KV head 1 changes only query heads 2 and 3 (G = 2): head h reads KV head h // G."""
    n, hq, hkv, d = 20, 4, 2, 8
    q, k, v = _rand(n, hq, hkv, d, 15)
    O1, _, _, _ = causal_attention(q, k, v)
    k2 = k.copy()
    k2[:, 1] *= -1.5
    O2, _, _, _ = causal_attention(q, k2, v)
    np.testing.assert_array_equal(O1[:, :2], O2[:, :2])
    assert np.abs(O1[:, 2:] - O2[:, 2:]).max() > 1e-3


def test_probs_match_library_softmax():
    """A from attention_probs equals torch's attention applied to V = identity."""
    n, hq, hkv, d = 24, 4, 2, 32
    q, k, _ = _rand(n, hq, hkv, d, 16)
    A = attention_probs(q, k)
    eye = np.tile(np.eye(n)[:, None, :], (1, hkv, 1))          # V = I: O row j is A row j
    vt = torch.from_numpy(np.ascontiguousarray(eye.transpose(1, 0, 2)))[None]
    ref = torch.nn.functional.scaled_dot_product_attention(_t(q), _t(k), vt, is_causal=True,
                                                           enable_gqa=True, scale=1 / math.sqrt(d))
    np.testing.assert_allclose(A, ref[0].numpy(), rtol=0, atol=1e-13)
