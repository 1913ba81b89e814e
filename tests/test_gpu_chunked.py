"""GPU parity of chunked prefill and prefix reuse (readings R25, R26) through the C ABI.

A chunk's rows are compared with the fp64 oracle's rows of the whole prompt; the window score
from the last chunk with the oracle's window score; the gather of cached blocks bit-exactly
with what was compacted; and a prompt that reuses another prompt's cached prefix (found by
the block-hash index) ends with the same compressed cache and the same outputs as the oracle
run on the whole prompt.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from oracle import prefix as oprefix
import workloads as wl
from tests._parity import (to_dev_bf16, bf16_to_f64, i32, assert_rows_close, assert_lse_close, assert_scores_close,
                           assert_keep_matches, gather_pools)

pytestmark = pytest.mark.gpu

kvs = pytest.importorskip("kv_cache_sparsification_amd")


def _say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    torch.cuda.set_device(0)


def _bits(rng, shape, scale=1.0):
    return wl.f32_to_bf16_bits((rng.standard_normal(shape) * scale).astype(np.float32))


@pytest.mark.parametrize("hq,hkv,d", [(4, 2, 64), (32, 8, 128), (16, 2, 64), (16, 1, 128)])
def test_chunk_rows_and_window_score(hq, hkv, d):
    """Three prompts, each with only its last m_s rows as queries (one is the whole prompt)."""
    _say(f"chunked prefill hq={hq} hkv={hkv} d={d}")
    rng = np.random.default_rng(d)
    n = [300, 1000, 517]
    m = [300, 256, 200]
    alpha = 32
    kb = [_bits(rng, (x, hkv, d)) for x in n]
    vb = [_bits(rng, (x, hkv, d)) for x in n]
    qb = [_bits(rng, (x, hq, d)) for x in n]
    for k_ in kb:
        k_[0, :, 3] = wl.f32_to_bf16_bits(np.float32([20.0] * hkv))   # a sink key
    cu_k = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(m)]).astype(np.int32)
    q_chunk = np.concatenate([q[x - mm:] for q, x, mm in zip(qb, n, m)])
    q, k, v = to_dev_bf16(q_chunk), to_dev_bf16(np.concatenate(kb)), to_dev_bf16(np.concatenate(vb))
    o, lse = kvs.kvs_prefill_attn_lse_chunk(q, k, v, i32(cu_q), i32(cu_k), max(m), max(n))
    S = kvs.kvs_window_score_chunk(q, k, lse, i32(cu_q), i32(cu_k), max(n), alpha)
    og, lg, Sg = bf16_to_f64(o), lse.cpu().numpy(), S.cpu().numpy().astype(np.float64)
    G = hq // hkv
    for s in range(3):
        qf, kf, vf = wl.bf16_bits_to_f64(qb[s]), wl.bf16_bits_to_f64(kb[s]), wl.bf16_bits_to_f64(vb[s])
        rows = range(n[s] - m[s], n[s])
        O_ref, lse_ref, _, _ = oracle.causal_attention(qf[n[s] - m[s]:], kf, vf, rows=rows, q_holds_rows=True)
        assert_rows_close(og[cu_q[s]:cu_q[s + 1]], O_ref, what=f"chunk O seq {s}")
        assert_lse_close(lg[:, cu_q[s]:cu_q[s + 1]], lse_ref, what=f"chunk LSE seq {s}")
        a = min(alpha, n[s])
        S_ref = oracle.window_score(qf[n[s] - a:], kf, lse_ref[:, m[s] - a:], alpha, window_only=True)
        assert_scores_close(Sg[:, cu_k[s]:cu_k[s + 1]], S_ref, what=f"chunk S seq {s}")


def test_gather_paged_round_trip():
    _say("gather paged")
    rng = np.random.default_rng(3)
    hkv, d = 8, 128
    n = [70, 33, 128]
    kb = np.concatenate([_bits(rng, (x, hkv, d)) for x in n])
    vb = np.concatenate([_bits(rng, (x, hkv, d)) for x in n])
    cu = np.concatenate([[0], np.cumsum(n)]).astype(np.int32)
    nb = 40
    perm = rng.permutation(nb)
    max_blocks = 8
    tables = np.full((3, max_blocks), -1, np.int32)
    used = 0
    for s, x in enumerate(n):
        c = -(-x // 16)
        tables[s, :c] = perm[used:used + c]
        used += c
    k_pool, v_pool = kvs.new_pools(nb, hkv, d)
    kvs.kvs_compact_paged(to_dev_bf16(kb), to_dev_bf16(vb), i32(cu), None, None, max(n), k_pool, v_pool,
                          i32(tables))
    counts = [x - 5 for x in n]                                         # a partial last block too
    dst = np.array([0, 100, 200], np.int32)
    k_out = torch.zeros(400, hkv, d, dtype=torch.bfloat16, device="cuda")
    v_out = torch.zeros_like(k_out)
    kvs.kvs_gather_paged(k_pool, v_pool, i32(tables), i32(counts), i32(dst), max(counts), k_out, v_out)
    ko = k_out.view(torch.int16).cpu().numpy().view(np.uint16)
    vo = v_out.view(torch.int16).cpu().numpy().view(np.uint16)
    for s in range(3):
        np.testing.assert_array_equal(ko[dst[s]:dst[s] + counts[s]], kb[cu[s]:cu[s] + counts[s]])
        np.testing.assert_array_equal(vo[dst[s]:dst[s] + counts[s]], vb[cu[s]:cu[s] + counts[s]])
        assert not ko[dst[s] + counts[s]:dst[s] + counts[s] + 3].any()   # nothing past the count


@pytest.mark.parametrize("k_budget", [None, 256])
def test_prefix_reuse_end_to_end(k_budget):
    """Prompt B shares its first 512 tokens with cached prompt A: the index finds them, B's K/V
    for them come back from A's blocks, only B's last rows are prefilled, and B's cache and
    outputs match the oracle run on the whole of B."""
    _say(f"prefix reuse, k_budget={k_budget}")
    rng = np.random.default_rng(17)
    hq, hkv, d, alpha = 32, 8, 128, 32
    nA, nB, shared = 800, 900, 512
    toks_a = rng.integers(0, 32000, nA)
    toks_b = np.concatenate([toks_a[:shared], rng.integers(0, 32000, nB - shared)])
    ka, va = _bits(rng, (nA, hkv, d)), _bits(rng, (nA, hkv, d))
    kbB = np.concatenate([ka[:shared], _bits(rng, (nB - shared, hkv, d))])   # same tokens, same K/V rows
    vbB = np.concatenate([va[:shared], _bits(rng, (nB - shared, hkv, d))])
    qbB = _bits(rng, (nB, hq, d))

    # A is cached in full (a full-cache layer's blocks) and registered by its block keys
    nb = 200
    alloc = kvs.BlockAllocator(nb, list(np.random.default_rng(2).permutation(nb)))
    k_pool, v_pool = kvs.new_pools(nb, hkv, d)
    k_pool.view(torch.int16).fill_(0x7FC0)
    v_pool.view(torch.int16).fill_(0x7FC0)
    table_a = alloc.alloc_n(-(-nA // 16))
    kvs.kvs_compact_paged(to_dev_bf16(ka), to_dev_bf16(va), i32([0, nA]), None, None, nA, k_pool, v_pool,
                          i32([table_a]))
    index = kvs.BlockHashIndex()
    index.register(0, toks_a)
    P, src = index.match(toks_b, alpha)
    assert (P, src) == oprefix_match(toks_a, toks_b, alpha)
    assert P == shared

    # B: the reused blocks come back from the pool, then B's own rows follow them
    k_all = torch.empty(nB, hkv, d, dtype=torch.bfloat16, device="cuda")
    v_all = torch.empty_like(k_all)
    shared_blocks = [table_a[bi] for _, bi in src]
    kvs.kvs_gather_paged(k_pool, v_pool, i32([shared_blocks]), i32([P]), i32([0]), P, k_all, v_all)
    k_all[P:] = to_dev_bf16(kbB[P:])
    v_all[P:] = to_dev_bf16(vbB[P:])
    q_rows = to_dev_bf16(qbB[P:])
    if k_budget is None:      # full layer: B keeps the shared blocks and writes its own rows after them
        for b in shared_blocks:
            alloc.incref(b)
        table_b = shared_blocks + alloc.alloc_n(-(-nB // 16) - len(shared_blocks))
    else:                     # compressed layer: B's selection goes to blocks of its own
        table_b = alloc.alloc_n(-(-k_budget // 16))
    res = kvs.prefill_compress_layer_chunked(q_rows, k_all, v_all, i32([0, nB - P]), i32([0, nB]), [nB - P], [nB],
                                             alpha, k_budget, k_pool, v_pool, [table_b], 64, cached=[P])
    qf, kf, vf = wl.bf16_bits_to_f64(qbB), wl.bf16_bits_to_f64(kbB), wl.bf16_bits_to_f64(vbB)
    O_ref, lse_ref, _, _ = oracle.causal_attention(qf[P:], kf, vf, rows=range(P, nB), q_holds_rows=True)
    assert_rows_close(bf16_to_f64(res["o"]), O_ref, what="B rows after the prefix")
    assert_lse_close(res["lse"].cpu().numpy(), lse_ref, what="B LSE")
    if k_budget is None:
        gk, gv = gather_pools(k_pool, v_pool, table_b, nB)
        np.testing.assert_array_equal(gk, kbB)
        np.testing.assert_array_equal(gv, vbB)
        ga, _ = gather_pools(k_pool, v_pool, table_a, nA)                # A's cache is untouched
        np.testing.assert_array_equal(ga, ka)
    else:
        _, lse_full, _, _ = oracle.causal_attention(qf, kf, vf, rows=range(nB - alpha, nB))
        S_ref = oracle.window_score(qf[nB - alpha:], kf, lse_full, alpha, window_only=True)
        S_g = res["scores"].cpu().numpy().astype(np.float64)
        assert_scores_close(S_g, S_ref, what="B scores")
        keep = res["keep_idx"].cpu().numpy().reshape(hkv, k_budget)
        gk, gv = gather_pools(k_pool, v_pool, table_b, k_budget)
        for g in range(hkv):
            np.testing.assert_array_equal(keep[g], oracle.select_keep(S_g[g], nB, alpha, k_budget))
            assert_keep_matches(keep[g], oracle.select_keep(S_ref[g], nB, alpha, k_budget), S_ref[g], nB, alpha,
                                k_budget, what=f"B keep head {g}")
            np.testing.assert_array_equal(gk[:, g], kbB[keep[g], g])
            np.testing.assert_array_equal(gv[:, g], vbB[keep[g], g])


def oprefix_match(toks_a, toks_b, alpha):
    idx = oprefix.PrefixIndex()
    idx.register(0, toks_a)
    return idx.match(toks_b, alpha)
