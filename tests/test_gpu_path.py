"""GPU parity of the HIP path against the fp64 oracle, through the C ABI.

Each test prints the case it is about to run (flushed) so a failing GPU step is named.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
import workloads as wl
from tests._parity import (to_dev_bf16, bf16_to_f64, bf16_bits, i32, assert_rows_close, assert_lse_close,
                           assert_scores_close, assert_keep_matches, gather_pools)

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


def _f64(bits):
    return wl.bf16_bits_to_f64(bits)


def run_full_path(w: wl.Workload, layer: int, check_decode_steps, decode_steps: int):
    """Prefill -> score -> top-k -> compaction -> decode for one single-sequence workload layer."""
    n = w.fixed_len
    k_budget = w.budgets[layer]
    G, alpha, d = w.g, w.alpha, w.d
    qb, kb, vb, cu = wl.prefill_batch(w, layer, [n])
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb)
    cu_d = i32(cu)
    qf, kf, vf = _f64(qb), _f64(kb), _f64(vb)

    # ---- step 1: prefill attention + LSE (+ row max and l)
    rowmax = torch.empty(w.hq, n, device="cuda", dtype=torch.float32)
    ell = torch.empty_like(rowmax)
    o, lse = kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, rowmax=rowmax, ell=ell)
    O_ref, lse_ref, m_ref, l_ref = oracle.causal_attention(qf, kf, vf)
    assert_rows_close(bf16_to_f64(o), O_ref, what="prefill O")
    lse_g = lse.cpu().numpy()
    assert_lse_close(lse_g, lse_ref)
    assert_lse_close(rowmax.cpu().numpy(), m_ref, what="rowmax")
    np.testing.assert_allclose(ell.cpu().numpy(), l_ref, rtol=1e-3, atol=0)
    # LSE = rowmax + ln(l) on the GPU side too
    np.testing.assert_allclose(lse_g, rowmax.cpu().numpy() + np.log(ell.cpu().numpy()), rtol=0, atol=1e-4)

    # ---- step 2: window score from the GPU's LSE
    S = kvs.kvs_window_score(q, k, lse, cu_d, n, alpha)
    S_ref = oracle.window_score(qf, kf, lse_ref, alpha)
    S_g = S.cpu().numpy().astype(np.float64)
    assert_scores_close(S_g, S_ref)
    np.testing.assert_allclose(S_g.sum(1), G * min(alpha, n), rtol=1e-4)   # each window row sums to one

    # ---- step 3: top-k
    k_eff = oracle.keep_count(n, k_budget)
    keep_off = i32([0, k_eff])
    keep = kvs.kvs_topk_select(S, cu_d, n, alpha, k_budget, keep_off, total_keep=k_eff)
    keep_g = keep.cpu().numpy().reshape(w.hkv, k_eff)
    for g in range(w.hkv):
        # same scores, same decision: bit-exact against the oracle fed the GPU's fp32 scores
        np.testing.assert_array_equal(keep_g[g], oracle.select_keep(S_g[g], n, alpha, k_budget))
        assert_keep_matches(keep_g[g], oracle.select_keep(S_ref[g], n, alpha, k_budget), S_ref[g], n, alpha,
                            k_budget, what=f"keep head {g}")

    # ---- step 4: compaction into blocks from the native allocator (pools poisoned with NaN)
    total_tokens = k_eff + decode_steps
    nblocks_needed = oracle.blocks_for(total_tokens)
    num_blocks = nblocks_needed + 13
    alloc = kvs.BlockAllocator(num_blocks, list(np.random.default_rng(5).permutation(num_blocks)))
    table = alloc.alloc_n(oracle.blocks_for(k_eff))
    max_blocks = nblocks_needed
    k_pool, v_pool = kvs.new_pools(num_blocks, w.hkv, d)
    k_pool.view(torch.int16).fill_(0x7FC0)
    v_pool.view(torch.int16).fill_(0x7FC0)
    tbl = np.full((1, max_blocks), -1, np.int32)
    tbl[0, :len(table)] = table
    kvs.kvs_compact_paged(k, v, cu_d, keep, keep_off, k_eff, k_pool, v_pool, i32(tbl))
    gk, gv = gather_pools(k_pool, v_pool, table, k_eff)
    for g in range(w.hkv):
        np.testing.assert_array_equal(gk[:, g], kb[keep_g[g], g])
        np.testing.assert_array_equal(gv[:, g], vb[keep_g[g], g])
    # the fused call (what the pipeline makes) leaves the same indices and pools
    k_pool2, v_pool2 = kvs.new_pools(num_blocks, w.hkv, d)
    k_pool2.view(torch.int16).fill_(0x7FC0)
    v_pool2.view(torch.int16).fill_(0x7FC0)
    keep2 = kvs.kvs_topk_compact(S, k, v, cu_d, n, alpha, k_budget, keep_off, k_pool2, v_pool2, i32(tbl),
                                 total_keep=k_eff)
    np.testing.assert_array_equal(keep2.cpu().numpy().reshape(w.hkv, k_eff), keep_g)
    assert torch.equal(k_pool2.view(torch.int16), k_pool.view(torch.int16))
    assert torch.equal(v_pool2.view(torch.int16), v_pool.view(torch.int16))
    del k_pool2, v_pool2

    # ---- step 5: decode steps with append (write-then-attend)
    cache_k = [kf[keep_g[g], g] for g in range(w.hkv)]
    cache_v = [vf[keep_g[g], g] for g in range(w.hkv)]
    ws = None
    for step in range(decode_steps):
        L = k_eff + step + 1
        if (L - 1) % 16 == 0:
            table.append(alloc.alloc())
            tbl[0, :len(table)] = table
        dq, dk, dv = wl.decode_step_inputs(w, layer, step, 1)
        ctx = i32([L])
        lse_d = torch.empty(1, w.hq, device="cuda", dtype=torch.float32)
        od = kvs.kvs_paged_decode(to_dev_bf16(dq), k_pool, v_pool, i32(tbl), ctx, L, new_k=to_dev_bf16(dk),
                                  new_v=to_dev_bf16(dv), lse=lse_d)
        for g in range(w.hkv):
            cache_k[g] = np.concatenate([cache_k[g], _f64(dk)[0, g][None]])
            cache_v[g] = np.concatenate([cache_v[g], _f64(dv)[0, g][None]])
        if step in check_decode_steps:
            kc = np.stack(cache_k, axis=1)
            vc = np.stack(cache_v, axis=1)
            o_ref, l_ref2 = oracle.decode_attention(_f64(dq)[0], kc, vc)
            assert_rows_close(bf16_to_f64(od)[0], o_ref, what=f"decode step {step}")
            assert_lse_close(lse_d.cpu().numpy()[0], l_ref2, what=f"decode lse step {step}")
    # the appended tokens landed in the pool
    gk, gv = gather_pools(k_pool, v_pool, table, k_eff + decode_steps)
    last_k = wl.decode_step_inputs(w, layer, decode_steps - 1, 1)[1]
    np.testing.assert_array_equal(gk[-1], last_k[0])
    return dict(keep=keep_g, S=S_g)


def test_tiny_workload_full_path():
    w = wl.WORKLOADS[1]
    _say("tiny workload: n=256 Hq=4 Hkv=2 d=64 alpha=16 k=64, 8 decode steps")
    out = run_full_path(w, 0, check_decode_steps=set(range(8)), decode_steps=8)
    # attention sink: token 0 is kept by every head
    assert all(0 in set(out["keep"][g]) for g in range(w.hkv))


def test_llama8b_layer_full_path():
    w = wl.WORKLOADS[2]
    _say("8B layer: n=4000 Hq=32 Hkv=8 d=128 alpha=32 k=400, 500 decode steps")
    out = run_full_path(w, 0, check_decode_steps={0, 1, 15, 16, 17, 100, 249, 250, 498, 499}, decode_steps=500)
    assert sum(0 in set(out["keep"][g]) for g in range(w.hkv)) >= 6


@pytest.mark.parametrize("hq,hkv,d,n,alpha,k", [(16, 2, 64, 600, 32, 96), (16, 1, 128, 777, 16, 64)])
def test_wide_groups_full_path(hq, hkv, d, n, alpha, k):
    """Groups of 8 and 16 query heads per KV head through every step: 256 window rows (two row
    chunks of the score), and decode plans of 8 wavefronts in one workgroup (d=64) and of
    4-wavefront splits with a merge (d=128)."""
    w = dataclasses.replace(wl.WORKLOADS[1], hq=hq, hkv=hkv, d=d, alpha=alpha, budgets=(k,), fixed_len=n,
                            decode_steps=20)
    _say(f"wide groups: n={n} Hq={hq} Hkv={hkv} d={d} alpha={alpha} k={k}, 20 decode steps")
    out = run_full_path(w, 0, check_decode_steps={0, 1, 2, 7, 11, 12, 19}, decode_steps=20)
    assert all(0 in set(out["keep"][g]) for g in range(hkv))


@pytest.mark.parametrize("d,hq,hkv", [(128, 8, 2), (64, 4, 4), (128, 16, 1), (64, 16, 2)])
def test_prefill_ragged_batch(d, hq, hkv):
    lengths = [1, 17, 130, 255, 64, 300, 256, 257, 513]
    _say(f"ragged prefill d={d} hq={hq} hkv={hkv} lengths={lengths}")
    r = np.random.default_rng(d + hq)
    T = sum(lengths)
    qb = wl.f32_to_bf16_bits(r.standard_normal((T, hq, d), dtype=np.float32))
    kb = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb)
    o, lse = kvs.kvs_prefill_attn_lse(q, k, v, i32(cu), max(lengths))
    og, lg = bf16_to_f64(o), lse.cpu().numpy()
    for s, n in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        O_ref, lse_ref, _, _ = oracle.causal_attention(_f64(qb[a:b]), _f64(kb[a:b]), _f64(vb[a:b]))
        assert_rows_close(og[a:b], O_ref, what=f"O seq {s}")
        assert_lse_close(lg[:, a:b], lse_ref, what=f"LSE seq {s}")
        # window score (alpha larger than some prompts) from the oracle's LSE fed to the GPU
    lse_ref_all = np.zeros((hq, T))
    for s, n in enumerate(lengths):
        a, b = cu[s], cu[s + 1]
        lse_ref_all[:, a:b] = oracle.causal_attention(_f64(qb[a:b]), _f64(kb[a:b]), _f64(vb[a:b]))[1]
    for alpha in (1, 16, 64):
        S = kvs.kvs_window_score(q, k, torch.from_numpy(lse_ref_all.astype(np.float32)).cuda(), i32(cu),
                                 max(lengths), alpha).cpu().numpy()
        lse32 = lse_ref_all.astype(np.float32).astype(np.float64)
        for s, n in enumerate(lengths):
            a, b = cu[s], cu[s + 1]
            S_ref = oracle.window_score(_f64(qb[a:b]), _f64(kb[a:b]), lse32[:, a:b], alpha)
            assert_scores_close(S[:, a:b].astype(np.float64), S_ref, what=f"S seq {s} a={alpha}")


def test_topk_exact_with_ties_and_budgets():
    """Constructed scores with many ties: the kernel's kept set equals the oracle's exactly."""
    r = np.random.default_rng(3)
    lengths = [5, 40, 600, 1000, 4097, 33, 20000]   # the last beyond the 16384 candidates held in LDS
    hkv = 3
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    S = (r.integers(0, 6, size=(hkv, T)) / 64.0).astype(np.float32)
    S[1] = r.random(T).astype(np.float32)                       # head 1: no ties
    S[2, :] = 0.25                                              # head 2: everything tied
    for alpha, kb in ((4, 4), (8, 30), (16, 512), (1, 2000)):
        _say(f"topk alpha={alpha} k={kb}")
        kept = [min(kb, n) for n in lengths]
        off = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
        keep = kvs.kvs_topk_select(torch.from_numpy(S).cuda(), i32(cu), max(lengths), alpha, kb, i32(off),
                                   total_keep=int(off[-1])).cpu().numpy()
        for s, n in enumerate(lengths):
            seg = keep[hkv * off[s]: hkv * off[s + 1]].reshape(hkv, kept[s])
            for g in range(hkv):
                ref = oracle.select_keep(S[g, cu[s]:cu[s + 1]].astype(np.float64), n, alpha, kb)
                np.testing.assert_array_equal(seg[g], ref, err_msg=f"seq {s} head {g} alpha {alpha} k {kb}")


@pytest.mark.parametrize("fused", [False, True])
def test_topk_over_score_ranges(fused):
    """Scores over very different ranges: all equal, differing only in their low bits, a few
    distinct values, zeros beside tiny positives, every exponent, and one binade (like the
    bench layer's non-sink scores); kept sets as the oracle's, for both entry points."""
    r = np.random.default_rng(41)
    n, alpha, kb, hkv = 3000, 16, 300, 6
    S = np.empty((hkv, n), np.float32)
    S[0] = 0.37                                                             # every score equal
    S[1] = (np.uint32(0x3D000000) | r.integers(0, 1 << 9, n).astype(np.uint32)).view(np.float32)   # 9 low bits
    S[2] = (r.integers(0, 5, n) * 0.125 + 1.0).astype(np.float32)           # five values
    S[3] = np.where(r.random(n) < 0.5, 0.0, r.random(n) * 1e-30).astype(np.float32)   # zeros and tiny ones
    S[4] = (2.0 ** r.uniform(-126, 6, n)).astype(np.float32)                # every exponent
    S[5] = (0.05 * (1 + 0.1 * r.standard_normal(n))).astype(np.float32)     # one binade
    _say(f"topk over score ranges, fused={fused}")
    S_d = torch.from_numpy(S).cuda()
    cu, off = i32([0, n]), i32([0, kb])
    if fused:
        k_src = torch.zeros(n, hkv, 64, device="cuda", dtype=torch.bfloat16)
        kp, vp = kvs.new_pools(-(-kb // 16), hkv, 64)
        tbl = i32([list(range(-(-kb // 16)))])
        keep = kvs.kvs_topk_compact(S_d, k_src, k_src, cu, n, alpha, kb, off, kp, vp, tbl, total_keep=kb)
    else:
        keep = kvs.kvs_topk_select(S_d, cu, n, alpha, kb, off, total_keep=kb)
    keep = keep.cpu().numpy().reshape(hkv, kb)
    for g in range(hkv):
        np.testing.assert_array_equal(keep[g], oracle.select_keep(S[g].astype(np.float64), n, alpha, kb),
                                      err_msg=f"head {g}")


def test_topk_threshold_bin_taken_whole():
    """The kept candidates are exactly the members of one radix bin (the top 11 bits, or the top
    22) above everything else: the search stops at that pass and must keep the same set."""
    r = np.random.default_rng(31)
    for n, alpha, kb in ((300, 8, 40), (4000, 32, 400), (20000, 16, 700)):
        kk = kb - alpha
        S = np.zeros((3, n), np.float32)
        pick = [r.choice(n - alpha, size=kk, replace=False) for _ in range(3)]
        S[:] = (r.random((3, n)) * 0.5).astype(np.float32)               # below the chosen ones
        S[0, pick[0]] = (1.0 + r.random(kk) * 0.24).astype(np.float32)     # one 11-bit bin: stops after one pass
        # head 1: the kept ones share their top 22 bits (low 10 bits differ); unkept scores of 1.5
        # share only their top 11, so the search stops after the second pass
        low = r.choice(1024, size=kk, replace=kk > 1024).astype(np.uint32)
        S[1, pick[1]] = (np.uint32(0x3FC00800) | low).view(np.float32)
        rest = np.setdiff1d(np.arange(n - alpha), pick[1])
        S[1, r.choice(rest, size=min(50, rest.size), replace=False)] = 1.5
        S[2, pick[2]] = 1.0                                                # one value, every copy kept
        _say(f"topk whole threshold bin n={n} alpha={alpha} k={kb}")
        keep = kvs.kvs_topk_select(torch.from_numpy(S).cuda(), i32([0, n]), n, alpha, kb, i32([0, kb]),
                                   total_keep=kb).cpu().numpy().reshape(3, kb)
        for g in range(3):
            ref = oracle.select_keep(S[g].astype(np.float64), n, alpha, kb)
            np.testing.assert_array_equal(keep[g], ref, err_msg=f"head {g} n {n}")
            np.testing.assert_array_equal(keep[g][:kk], np.sort(pick[g]))


def test_compaction_offsets_keep_all_and_partial_blocks():
    _say("compaction with misaligned destination offsets, keep-all and partial blocks")
    r = np.random.default_rng(4)
    lengths = [3, 16, 33, 70]
    hkv, d = 2, 128
    T = sum(lengths)
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    kb = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    offs = [0, 5, 16, 31]
    nb = 64
    k_pool, v_pool = kvs.new_pools(nb, hkv, d)
    k_pool.view(torch.int16).fill_(0x7FC0)
    v_pool.view(torch.int16).fill_(0x7FC0)
    perm = list(r.permutation(nb))
    max_blocks = 8
    tbl = np.full((len(lengths), max_blocks), -1, np.int32)
    tables = []
    for s, n in enumerate(lengths):
        t = [perm.pop() for _ in range(oracle.blocks_for(offs[s] + n))]
        tables.append(t)
        tbl[s, :len(t)] = t
    kvs.kvs_compact_paged(to_dev_bf16(kb), to_dev_bf16(vb), i32(cu), None, None, max(lengths), k_pool, v_pool,
                          i32(tbl), dst_slot_offset=i32(offs))
    for s, n in enumerate(lengths):
        gk, gv = gather_pools(k_pool, v_pool, tables[s], offs[s] + n)
        np.testing.assert_array_equal(gk[offs[s]:], kb[cu[s]:cu[s + 1]])
        np.testing.assert_array_equal(gv[offs[s]:], vb[cu[s]:cu[s + 1]])
        assert np.all(gk[:offs[s]] == 0x7FC0) and np.all(gv[:offs[s]] == 0x7FC0)   # earlier slots untouched


@pytest.mark.parametrize("d,hq,hkv,lens", [(128, 32, 8, [5000, 1, 17, 900]), (64, 4, 2, [3, 2000]),
                                           (128, 8, 8, [16, 32, 48]), (64, 16, 2, [700, 5]),
                                           (64, 16, 1, [300, 2500]), (128, 16, 1, [1200, 7]),
                                           (128, 32, 8, [100000, 3]),    # 6250 blocks: the split count is capped
                                           # wide batches of short contexts (one workgroup per sequence
                                           # and head, several rounds) and a mid-size split plan
                                           (128, 32, 8, list(range(400, 700, 15))),
                                           (128, 32, 8, list(range(250, 390, 7))),
                                           (128, 32, 8, [3000 + 33 * i for i in range(4)]),
                                           (128, 32, 8, [16400, 16399, 17000, 16384])])   # the long-context plan
def test_decode_batch_splits_and_merge(d, hq, hkv, lens):
    """Full-cache decode over several contexts, with and without append; long contexts split and merge."""
    _say(f"decode batch d={d} hq={hq} hkv={hkv} lens={lens}")
    r = np.random.default_rng(d + len(lens))
    B = len(lens)
    max_ctx = max(lens)
    max_blocks = oracle.blocks_for(max_ctx)
    nb = B * max_blocks + 5
    perm = list(r.permutation(nb))
    k_pool, v_pool = kvs.new_pools(nb, hkv, d)
    k_pool.view(torch.int16).fill_(0x7FC0)
    v_pool.view(torch.int16).fill_(0x7FC0)
    tbl = np.full((B, max_blocks), -1, np.int32)
    caches = []
    for b, L in enumerate(lens):
        t = [perm.pop() for _ in range(oracle.blocks_for(L))]
        tbl[b, :len(t)] = t
        kc = wl.f32_to_bf16_bits(r.standard_normal((L, hkv, d), dtype=np.float32))
        vc = wl.f32_to_bf16_bits(r.standard_normal((L, hkv, d), dtype=np.float32))
        cu = i32([0, L])
        # all L slots; the append case then overwrites slot L-1
        kvs.kvs_compact_paged(to_dev_bf16(kc), to_dev_bf16(vc), cu, None, None, L, k_pool, v_pool, i32(tbl[b:b + 1]))
        caches.append((kc, vc))
    qb = wl.f32_to_bf16_bits(r.standard_normal((B, hq, d), dtype=np.float32))
    nk = wl.f32_to_bf16_bits(r.standard_normal((B, hkv, d), dtype=np.float32))
    nv = wl.f32_to_bf16_bits(r.standard_normal((B, hkv, d), dtype=np.float32))
    ctx = i32(lens)
    for append in (False, True):
        lse = torch.empty(B, hq, device="cuda", dtype=torch.float32)
        o = kvs.kvs_paged_decode(to_dev_bf16(qb), k_pool, v_pool, i32(tbl), ctx, max_ctx,
                                 new_k=to_dev_bf16(nk) if append else None, new_v=to_dev_bf16(nv) if append else None,
                                 lse=lse)
        og, lg = bf16_to_f64(o), lse.cpu().numpy()
        for b, L in enumerate(lens):
            kc, vc = _f64(caches[b][0]), _f64(caches[b][1])
            if append:
                kc[L - 1], vc[L - 1] = _f64(nk[b]), _f64(nv[b])
            o_ref, l_ref = oracle.decode_attention(_f64(qb[b]), kc, vc)
            assert_rows_close(og[b], o_ref, what=f"decode b={b} append={append}")
            assert_lse_close(lg[b], l_ref, what=f"decode lse b={b} append={append}")


def _contexts_by_split_count(batch, hq, hkv, d, wanted, limit):
    """For each wanted split count, the shortest context (up to limit) whose launch plan has it,
    read back through the workspace size (batch * hq * splits * (d + 2) fp32 partials)."""
    found = {}
    for L in range(1, limit + 1):
        ws = kvs.kvs_paged_decode_workspace_size(batch, hq, hkv, d, L)
        s = ws // (batch * hq * (d + 2) * 4) if ws else 1
        if s in wanted and s not in found:
            found[s] = L
    return found


@pytest.mark.parametrize("d,hq,hkv", [(128, 32, 8), (64, 16, 2)])
def test_decode_merge_fetch_widths(d, hq, hkv):
    """The merge kernel fetches 4, 8, 12 or 16 splits per round trip, the fewest covering the
    launch's split count, and loops past 16: contexts at both sides of every width's edge."""
    wanted = {2, 3, 4, 5, 8, 9, 12, 13, 16, 17, 33}
    found = _contexts_by_split_count(1, hq, hkv, d, wanted, 6000)
    _say(f"merge widths d={d}: split count -> context {sorted(found.items())}")
    assert {4, 5, 8, 9, 12, 13, 16, 17} <= set(found), found
    for s, L in sorted(found.items()):
        test_decode_batch_splits_and_merge(d, hq, hkv, [L])
        test_decode_batch_splits_and_merge(d, hq, hkv, [L, max(1, L // 3)])   # a shorter second context


@pytest.mark.parametrize("lens,hkv,d,alpha,kb,offs,ties", [
    ([4000], 8, 128, 32, 400, None, False),                    # the 8B layer's shape
    ([300, 17, 1000, 5, 0, 64], 2, 64, 16, 64, [3, 0, 17, 9, 0, 15], False),   # ragged, keep-all, empty, offsets
    ([900, 33], 4, 128, 32, 32, None, False),                   # the budget is the window
    ([2000, 1500], 2, 128, 8, 300, [5, 16], True),              # many equal scores
    ([16000], 1, 64, 32, 700, None, False),                     # the most candidates the fused form takes
    ([600] * 20, 2, 128, 32, 512, None, False),                 # wide batch: the two kernels run instead
    ([20000], 2, 64, 32, 700, None, False),                     # candidates beyond the LDS: two kernels
    ([20000], 1, 64, 32, 17000, [7], False)])                   # kept list beyond the LDS: two kernels
def test_topk_compact_matches_separate_calls(lens, hkv, d, alpha, kb, offs, ties):
    """The fused selection-and-compaction call against kvs_topk_select followed by
    kvs_compact_paged: the same kept indices and the same pools, bit for bit (pools poisoned
    with NaN first, so a slot written by one and not the other shows)."""
    _say(f"topk_compact lens={lens} hkv={hkv} d={d} alpha={alpha} k={kb} offs={offs} ties={ties}")
    r = np.random.default_rng(sum(lens) + kb)
    T = sum(lens)
    S = r.random((hkv, T), dtype=np.float32)
    if ties:
        S = np.round(S * 8) / 8                  # 9 distinct values
    kk = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    vv = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    kept = [min(kb, n) for n in lens]
    koff = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    o = offs or [0] * len(lens)
    nbs = [-(-(o[i] + kept[i]) // 16) for i in range(len(lens))]
    nb = sum(nbs) + 3
    perm = r.permutation(nb)
    tbl = np.full((len(lens), max(max(nbs), 1)), -1, np.int32)
    at = 0
    for i, c in enumerate(nbs):
        tbl[i, :c] = perm[at:at + c]
        at += c
    S_d, k_d, v_d = torch.from_numpy(S).cuda(), to_dev_bf16(kk), to_dev_bf16(vv)
    cu_d, koff_d, tbl_d = i32(cu), i32(koff), i32(tbl)
    off_d = i32(offs) if offs is not None else None
    res = []
    for fused in (False, True):
        kp, vp = kvs.new_pools(nb, hkv, d)
        kp.view(torch.int16).fill_(0x7FC0)
        vp.view(torch.int16).fill_(0x7FC0)
        if fused:
            keep = kvs.kvs_topk_compact(S_d, k_d, v_d, cu_d, max(lens), alpha, kb, koff_d, kp, vp, tbl_d,
                                        total_keep=int(koff[-1]), dst_slot_offset=off_d)
        else:
            keep = kvs.kvs_topk_select(S_d, cu_d, max(lens), alpha, kb, koff_d, total_keep=int(koff[-1]))
            kvs.kvs_compact_paged(k_d, v_d, cu_d, keep, koff_d, max(kept), kp, vp, tbl_d, dst_slot_offset=off_d)
        torch.cuda.synchronize()
        res.append((keep.cpu().numpy(), bf16_bits(kp), bf16_bits(vp)))
    for what, a, b in zip(("keep_idx", "K pool", "V pool"), res[0], res[1]):
        np.testing.assert_array_equal(b, a, err_msg=f"{what}: fused against separate calls")
    # and the kept sets are the oracle's (ties to the lower index)
    for s_, n in enumerate(lens):
        for g in range(hkv):
            if n == 0:
                continue
            got = res[1][0][hkv * koff[s_] + g * kept[s_]: hkv * koff[s_] + (g + 1) * kept[s_]]
            ref = oracle.select_keep(S[g, cu[s_]:cu[s_ + 1]].astype(np.float64), n, alpha, kb)
            np.testing.assert_array_equal(got, ref, err_msg=f"keep prompt {s_} head {g}")


def test_copy_blocks_for_copy_on_write():
    _say("copy_blocks")
    hkv, d, nb = 2, 128, 10
    k_pool, v_pool = kvs.new_pools(nb, hkv, d)
    k_pool.copy_(torch.randn(k_pool.shape, device="cuda").to(torch.bfloat16))
    v_pool.copy_(torch.randn(v_pool.shape, device="cuda").to(torch.bfloat16))
    before_k, before_v = k_pool.clone(), v_pool.clone()
    pairs = i32([[1, 7], [4, 2], [9, 0]])
    kvs.kvs_copy_blocks(k_pool, v_pool, pairs)
    torch.cuda.synchronize()
    for s, t in ((1, 7), (4, 2), (9, 0)):
        assert torch.equal(k_pool[t].view(torch.int16), before_k[s].view(torch.int16))
        assert torch.equal(v_pool[t].view(torch.int16), before_v[s].view(torch.int16))
    for untouched in (1, 3, 4, 5, 6, 8, 9):
        assert torch.equal(k_pool[untouched].view(torch.int16), before_k[untouched].view(torch.int16))


def test_single_token_and_window_only():
    """n = 1 prompt; budget equal to the window."""
    _say("n=1 and k == alpha")
    r = np.random.default_rng(9)
    hq, hkv, d = 4, 2, 64
    for n, alpha, kb in ((1, 4, 4), (50, 8, 8)):
        qb = wl.f32_to_bf16_bits(r.standard_normal((n, hq, d), dtype=np.float32))
        kk = wl.f32_to_bf16_bits(r.standard_normal((n, hkv, d), dtype=np.float32))
        vb = wl.f32_to_bf16_bits(r.standard_normal((n, hkv, d), dtype=np.float32))
        q, k, v = to_dev_bf16(qb), to_dev_bf16(kk), to_dev_bf16(vb)
        cu = i32([0, n])
        o, lse = kvs.kvs_prefill_attn_lse(q, k, v, cu, n)
        O_ref, lse_ref, _, _ = oracle.causal_attention(_f64(qb), _f64(kk), _f64(vb))
        assert_rows_close(bf16_to_f64(o), O_ref)
        S = kvs.kvs_window_score(q, k, lse, cu, n, alpha)
        k_eff = min(kb, n)
        keep = kvs.kvs_topk_select(S, cu, n, alpha, kb, i32([0, k_eff]), total_keep=k_eff).cpu().numpy()
        for g in range(hkv):
            np.testing.assert_array_equal(keep[g * k_eff:(g + 1) * k_eff], np.arange(n - k_eff, n))


@pytest.mark.parametrize("fp8", [False, True])
@pytest.mark.parametrize("d,hq,hkv,lens", [(128, 32, 8, [32, 17, 1, 400]), (64, 4, 2, [16, 3000])])
def test_decode_ignores_unwritten_slots(fp8, d, hq, hkv, lens):
    """Slots past the context in a sequence's last block were never written and may hold any bit
    pattern: here NaN (and NaN codes and scales in the 8-bit cache).  Masked scores give P = 0,
    which does not cancel a NaN in the P.V product, so the kernel must keep those values out.
    Covers contexts ending mid-block and an appended token that opens a fresh block."""
    _say(f"decode over NaN-filled tails fp8={fp8} d={d} hq={hq} hkv={hkv} lens={lens}")
    from oracle import fp8 as ofp8
    r = np.random.default_rng(d + 7 * len(lens) + fp8)
    B = len(lens)
    max_ctx = max(lens) + 1
    max_blocks = oracle.blocks_for(max_ctx)
    nb = B * max_blocks + 3
    perm = list(r.permutation(nb))
    tbl = np.full((B, max_blocks), -1, np.int32)
    for b, L in enumerate(lens):
        t = [perm.pop() for _ in range(oracle.blocks_for(L + 1))]
        tbl[b, :len(t)] = t
    pools = kvs.new_pools_fp8(nb, hkv, d) if fp8 else kvs.new_pools(nb, hkv, d)
    caches = []
    for b, L in enumerate(lens):
        kc = wl.f32_to_bf16_bits(r.standard_normal((L, hkv, d), dtype=np.float32))
        vc = wl.f32_to_bf16_bits(r.standard_normal((L, hkv, d), dtype=np.float32))
        compact = kvs.kvs_compact_paged_fp8 if fp8 else kvs.kvs_compact_paged
        compact(to_dev_bf16(kc), to_dev_bf16(vc), i32([0, L]), None, None, L, *pools, i32(tbl[b:b + 1]))
        caches.append((kc, vc))
    torch.cuda.synchronize()
    # every slot at or past each context, in the sequence's blocks, as never written: NaN
    for b, L in enumerate(lens):
        for p in range(L, oracle.blocks_for(L + 1) * 16):
            blk, slot = int(tbl[b, p // 16]), p % 16
            if fp8:
                pools[0][blk, :, slot, :] = 0x7F
                pools[1][blk, :, :, slot] = 0x7F
                pools[2][blk, :, slot] = float("nan")
                pools[3][blk, :, slot] = float("nan")
            else:
                pools[0][blk, :, slot, :].view(torch.int16).fill_(0x7FC0)
                pools[1][blk, :, :, slot].view(torch.int16).fill_(0x7FC0)
    qb = wl.f32_to_bf16_bits(r.standard_normal((B, hq, d), dtype=np.float32))
    nk = wl.f32_to_bf16_bits(r.standard_normal((B, hkv, d), dtype=np.float32))
    nv = wl.f32_to_bf16_bits(r.standard_normal((B, hkv, d), dtype=np.float32))
    cached = lambda x: ofp8.dequantize_rows(*ofp8.quantize_rows(x)) if fp8 else x
    decode = kvs.kvs_paged_decode_fp8 if fp8 else kvs.kvs_paged_decode
    for append in (False, True):   # L = len (the tail after it is NaN), then len + 1 with the new token
        ctx = i32([L + append for L in lens])
        lse = torch.empty(B, hq, device="cuda", dtype=torch.float32)
        o = decode(to_dev_bf16(qb), *pools, i32(tbl), ctx, max_ctx, new_k=to_dev_bf16(nk) if append else None,
                   new_v=to_dev_bf16(nv) if append else None, lse=lse)
        og, lg = bf16_to_f64(o), lse.cpu().numpy()
        assert np.isfinite(og).all() and np.isfinite(lg).all()
        for b, L in enumerate(lens):
            kc, vc = cached(_f64(caches[b][0])), cached(_f64(caches[b][1]))
            if append:
                kc = np.concatenate([kc, cached(_f64(nk[b:b + 1]))])
                vc = np.concatenate([vc, cached(_f64(nv[b:b + 1]))])
            o_ref, l_ref = oracle.decode_attention(_f64(qb[b]), kc, vc)
            assert_rows_close(og[b], o_ref, what=f"decode b={b} append={append}")
            assert_lse_close(lg[b], l_ref, what=f"decode lse b={b} append={append}")


def test_prefill_without_statistics_writes_only_o():
    """With the LSE output left out (the unmodified attention, measured against the one that
    returns its statistics) the call runs and O is bit-identical."""
    w = wl.WORKLOADS[2]
    n = 1000
    _say(f"prefill without LSE: n={n}, 32/8 heads, d=128")
    qb, kb, vb, cu = wl.prefill_batch(w, 0, [n])
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kb), to_dev_bf16(vb)
    cu_d = i32(cu)
    o1, lse = kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n)
    o2, none = kvs.kvs_prefill_attn_lse(q, k, v, cu_d, n, skip_lse=True)
    torch.cuda.synchronize()
    assert none is None
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16))


@pytest.mark.parametrize("n,d", [(1000, 128), (20, 64), (777, 64)])
def test_single_prompt_matches_batched_form(n, d):
    """A prompt alone and the same prompt followed by an empty one (a different grid and work
    mapping): prefill, window score and top-k give the same bits."""
    hq, hkv, alpha, kb = 8, 2, 32, 200
    _say(f"single prompt against the batched form: n={n} d={d}")
    r = np.random.default_rng(n + d)
    qb = wl.f32_to_bf16_bits(r.standard_normal((n, hq, d), dtype=np.float32))
    kk = wl.f32_to_bf16_bits(r.standard_normal((n, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(r.standard_normal((n, hkv, d), dtype=np.float32))
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kk), to_dev_bf16(vb)
    ke = min(kb, n)
    outs = []
    for cu, koff in (([0, n], [0, ke]), ([0, n, n], [0, ke, ke])):
        o, lse = kvs.kvs_prefill_attn_lse(q, k, v, i32(cu), n)
        S = kvs.kvs_window_score(q, k, lse, i32(cu), n, alpha)
        keep = kvs.kvs_topk_select(S, i32(cu), n, alpha, kb, i32(koff), total_keep=ke)
        torch.cuda.synchronize()
        outs.append((bf16_bits(o), lse.cpu().numpy().view(np.uint32), S.cpu().numpy().view(np.uint32),
                     keep.cpu().numpy()))
    for what, a, b in zip(("O", "LSE", "S", "keep"), outs[0], outs[1]):
        np.testing.assert_array_equal(a, b, err_msg=f"{what}: one prompt against the batched form")
    O_ref, lse_ref, _, _ = oracle.causal_attention(_f64(qb), _f64(kk), _f64(vb))
    assert_rows_close(bf16_to_f64(torch.from_numpy(outs[0][0].view(np.int16)).view(torch.bfloat16)), O_ref)
    assert_lse_close(outs[0][1].view(np.float32), lse_ref)


def test_empty_prompts_in_a_ragged_batch():
    """Prompts of length 0 between real ones (repeated cu_seqlens entries): they produce no
    rows, scores, kept indices or blocks, and the prompts around them match the oracle."""
    lengths = [0, 7, 0, 300, 0, 40, 0]
    hq, hkv, d, alpha, kb = 8, 2, 128, 16, 32
    _say(f"empty prompts in a ragged batch: lengths={lengths}")
    r = np.random.default_rng(23)
    T = sum(lengths)
    qb = wl.f32_to_bf16_bits(r.standard_normal((T, hq, d), dtype=np.float32))
    kk = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    vb = wl.f32_to_bf16_bits(r.standard_normal((T, hkv, d), dtype=np.float32))
    cu = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    q, k, v = to_dev_bf16(qb), to_dev_bf16(kk), to_dev_bf16(vb)
    o, lse = kvs.kvs_prefill_attn_lse(q, k, v, i32(cu), max(lengths))
    S = kvs.kvs_window_score(q, k, lse, i32(cu), max(lengths), alpha)
    kept = [min(kb, n) for n in lengths]
    koff = np.concatenate([[0], np.cumsum(kept)]).astype(np.int32)
    keep = kvs.kvs_topk_select(S, i32(cu), max(lengths), alpha, kb, i32(koff), total_keep=int(koff[-1]))
    nbs = [-(-c // 16) for c in kept]
    k_pool, v_pool = kvs.new_pools(sum(nbs) + 1, hkv, d)
    k_pool.view(torch.int16).fill_(0x7FC0)
    v_pool.view(torch.int16).fill_(0x7FC0)
    tbl = np.full((len(lengths), max(nbs)), -1, np.int32)
    at = 0
    for s, nb in enumerate(nbs):
        tbl[s, :nb] = np.arange(at, at + nb)
        at += nb
    kvs.kvs_compact_paged(k, v, i32(cu), keep, i32(koff), max(kept), k_pool, v_pool, i32(tbl))
    torch.cuda.synchronize()
    og, lg, Sg, keepg = bf16_to_f64(o), lse.cpu().numpy(), S.cpu().numpy().astype(np.float64), keep.cpu().numpy()
    assert keepg.size == hkv * koff[-1]
    kbits, vbits = bf16_bits(k), bf16_bits(v)
    for s, n in enumerate(lengths):
        if n == 0:
            continue
        a, b = cu[s], cu[s + 1]
        O_ref, lse_ref, _, _ = oracle.causal_attention(_f64(qb[a:b]), _f64(kk[a:b]), _f64(vb[a:b]))
        assert_rows_close(og[a:b], O_ref, what=f"O seq {s}")
        assert_lse_close(lg[:, a:b], lse_ref, what=f"LSE seq {s}")
        S_ref = oracle.window_score(_f64(qb[a:b]), _f64(kk[a:b]), lse_ref, alpha)
        assert_scores_close(Sg[:, a:b], S_ref, what=f"S seq {s}")
        seg = keepg[hkv * koff[s]: hkv * koff[s + 1]].reshape(hkv, kept[s])
        for g in range(hkv):
            np.testing.assert_array_equal(seg[g], oracle.select_keep(Sg[g, a:b], n, alpha, kb))
        gk, gv = gather_pools(k_pool, v_pool, tbl[s, :nbs[s]], kept[s])
        for g in range(hkv):
            np.testing.assert_array_equal(gk[:, g], kbits[a + seg[g], g])
            np.testing.assert_array_equal(gv[:, g], vbits[a + seg[g], g])
    # the spare block was never written
    assert torch.all(k_pool[-1].view(torch.int16) == 0x7FC0)
