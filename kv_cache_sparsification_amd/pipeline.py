"""Host orchestration of one layer's prefill-and-compress step (no device readback).

[KVS] Novita AI, "How KV Sparsity Achieves 1.5x Acceleration for vLLM", Key techniques 1
(step preparation): the first three layers keep a full cache, later layers keep a budget
k_l per head; [KVS] Key techniques 2: rowmax/l from the attention feed the window score,
whose top-k_l tokens are kept.  [PAG] Ultralytics glossary, "PagedAttention", "How paging
works": blocks come from the allocator's free list and a table records their order.

Every size the kernels need (k_eff = min(k_l, n) per prompt, the keep offsets, the number
of blocks) follows from the prompt lengths, the budget and the window on the host, so the
host never waits for the device.
"""
from __future__ import annotations

import math
from typing import List, Optional, Sequence

import torch

from ._lib import BLOCK_SIZE
from . import ops

FULL_CACHE_LAYERS = 3   # [KVS] Key techniques 1: the first three layers store every KV


def layer_policy(layer: int, k_budget: Optional[int], full_layers: int = FULL_CACHE_LAYERS) -> Optional[int]:
    """The budget a layer compresses to, or None for a full-cache layer."""
    return None if layer < full_layers else k_budget


def keep_counts(lengths: Sequence[int], k_budget: Optional[int]) -> List[int]:
    """Tokens each prompt keeps per KV head: n for a full layer, else min(k_l, n)."""
    return [n if (k_budget is None or k_budget >= n) else k_budget for n in lengths]


def blocks_needed(tokens: int) -> int:
    return -(-tokens // BLOCK_SIZE)


def prefill_compress_layer(q, k, v, cu_seqlens, lengths: Sequence[int], alpha: int, k_budget: Optional[int],
                           allocator, k_pool, v_pool, max_blocks: int, scale: Optional[float] = None,
                           tables: Optional[List[List[int]]] = None, stream=None):
    """Run prefill attention + (window score + top-k when compressing) + compaction for one layer.

    lengths are the host copies of the prompt lengths; tables (host lists) may be given to
    reuse blocks, else ceil(k_eff / 16) blocks per prompt are taken from the allocator.
    Returns a dict with o, lse, scores, keep_idx, keep_offsets, tables and the device tables.
    """
    dev = q.device
    max_n = max(lengths)
    o, lse = ops.kvs_prefill_attn_lse(q, k, v, cu_seqlens, max_n, scale=scale, stream=stream)
    kept = keep_counts(lengths, k_budget)
    if tables is None:
        tables = [allocator.alloc_n(blocks_needed(c)) for c in kept]
    tbl = torch.full((len(lengths), max_blocks), -1, dtype=torch.int32)
    for i, t in enumerate(tables):
        if len(t) > max_blocks:
            raise ValueError("block table longer than max_blocks")
        tbl[i, :len(t)] = torch.tensor(t, dtype=torch.int32)
    tbl_dev = tbl.to(dev, non_blocking=False)
    scores = keep_idx = keep_off_dev = None
    if k_budget is None:
        ops.kvs_compact_paged(k, v, cu_seqlens, None, None, max(kept), k_pool, v_pool, tbl_dev, stream=stream)
    else:
        scores = ops.kvs_window_score(q, k, lse, cu_seqlens, max_n, alpha, scale=scale, stream=stream)
        keep_off = [0]
        for c in kept:
            keep_off.append(keep_off[-1] + c)
        keep_off_dev = torch.tensor(keep_off, dtype=torch.int32).to(dev)
        keep_idx = ops.kvs_topk_compact(scores, k, v, cu_seqlens, max_n, alpha, k_budget, keep_off_dev, k_pool,
                                        v_pool, tbl_dev, total_keep=keep_off[-1], stream=stream)
    return dict(o=o, lse=lse, scores=scores, keep_idx=keep_idx, keep_offsets=keep_off_dev, kept=kept,
                tables=tables, tables_dev=tbl_dev)


def default_scale(d: int) -> float:
    return 1.0 / math.sqrt(d)


def check_chunk_lengths(q_lengths: Sequence[int], k_lengths: Sequence[int], alpha: int, scored: bool) -> None:
    """Host check of a chunked step's lengths (see prefill_compress_layer_chunked)."""
    if len(q_lengths) != len(k_lengths):
        raise ValueError("q_lengths and k_lengths differ in length")
    for s, (m, n) in enumerate(zip(q_lengths, k_lengths)):
        if m < 0 or m > n:
            raise ValueError(f"prompt {s}: chunk of {m} rows for a prompt of {n} tokens")
        if scored and m < min(alpha, n):
            raise ValueError(f"prompt {s}: the chunk holds {m} rows but the window score needs the last "
                             f"{min(alpha, n)}")


def prefill_compress_layer_chunked(q, k, v, cu_q, cu_k, q_lengths: Sequence[int], k_lengths: Sequence[int],
                                   alpha: int, k_budget: Optional[int], k_pool, v_pool, tables: List[List[int]],
                                   max_blocks: int, cached: Optional[Sequence[int]] = None,
                                   scale: Optional[float] = None, stream=None):
    """One layer's step for prompts whose query rows are only their last q_lengths[s] rows (a
    chunk, or everything after a reused prefix); k/v hold all k_lengths[s] tokens.

    Compressed layers select over all n_s tokens and compact into `tables` from slot 0; a full
    layer writes only rows cached[s] .. n_s-1 (the reused prefix keeps its shared blocks), from
    slot cached[s].  Returns o, lse (chunk rows), scores, keep_idx, keep_offsets, tables_dev.

    Raises ValueError before any launch when a prompt's chunk is longer than the prompt, or, in a
    compressed layer, holds fewer than its last min(alpha, n) rows: the window score reads the
    LSE of the window rows from the chunk, and rows before it would silently be left out.
    """
    check_chunk_lengths(q_lengths, k_lengths, alpha, k_budget is not None)
    dev = q.device
    max_q, max_k = max(q_lengths), max(k_lengths)
    o, lse = ops.kvs_prefill_attn_lse_chunk(q, k, v, cu_q, cu_k, max_q, max_k, scale=scale, stream=stream)
    tbl = torch.full((len(k_lengths), max_blocks), -1, dtype=torch.int32)
    for i, t in enumerate(tables):
        if len(t) > max_blocks:
            raise ValueError("block table longer than max_blocks")
        tbl[i, :len(t)] = torch.tensor(t, dtype=torch.int32)
    tbl_dev = tbl.to(dev)
    scores = keep_idx = None
    if k_budget is None:
        cached = [0] * len(k_lengths) if cached is None else list(cached)
        kept = [n - c for n, c in zip(k_lengths, cached)]
        # every head keeps rows cached[s] .. n_s-1, in order
        keep = torch.cat([torch.arange(c, n, dtype=torch.int32).repeat(k.shape[1])
                          for c, n in zip(cached, k_lengths)]).to(dev)
        keep_off = [0]
        for c in kept:
            keep_off.append(keep_off[-1] + c)
        keep_off_dev = torch.tensor(keep_off, dtype=torch.int32).to(dev)
        ops.kvs_compact_paged(k, v, cu_k, keep, keep_off_dev, max(kept), k_pool, v_pool, tbl_dev,
                              dst_slot_offset=torch.tensor(cached, dtype=torch.int32).to(dev), stream=stream)
        keep_idx = keep
    else:
        kept = keep_counts(k_lengths, k_budget)
        scores = ops.kvs_window_score_chunk(q, k, lse, cu_q, cu_k, max_k, alpha, scale=scale, stream=stream)
        keep_off = [0]
        for c in kept:
            keep_off.append(keep_off[-1] + c)
        keep_off_dev = torch.tensor(keep_off, dtype=torch.int32).to(dev)
        keep_idx = ops.kvs_topk_compact(scores, k, v, cu_k, max_k, alpha, k_budget, keep_off_dev, k_pool, v_pool,
                                        tbl_dev, total_keep=keep_off[-1], stream=stream)
    return dict(o=o, lse=lse, scores=scores, keep_idx=keep_idx, keep_offsets=keep_off_dev, kept=kept,
                tables_dev=tbl_dev)


def prefix_rows_reused(cache, layer: int, plan, n: int, alpha: int) -> int:
    """Prompt rows a new member reads back from its group's prefix blocks in `layer` instead of
    computing them.

    [PAG] "Sharing blocks between sequences": sequences of one prefix map the same blocks.  A
    member reuses the whole prefix when the layer carries the group's prefix, the prefix was
    written before this member's admission (a member whose admission created it computes it),
    and the member's own rows still hold its last min(alpha, n) tokens, whose LSE the window
    score reads.  Otherwise 0: the member computes all its rows.
    """
    P = cache.prefix_len
    if P and n > P and cache.carries_prefix(layer) and not plan.new_prefix and n - P >= min(alpha, n):
        return P
    return 0


def prefill_compress_admission(cache, layer: int, seqs: Sequence, plans, q, k, v, alpha: int, k_pool, v_pool,
                               scale: Optional[float] = None, stream=None):
    """One layer of an admission wave under continuous batching with shared prefixes.

    seqs: the admitted prompts in batch order as (seq_id, group, n); plans: {seq_id: the list
    cache.admit() returned}.  q holds the rows each prompt computes (rows r0..n-1 with
    r0 = prefix_rows_reused(...)), k and v all n rows of every prompt; the rows of a reused
    prefix are overwritten here by the read-back from the group's blocks.  In order, on the
    caller's stream and with no device readback:
      1. a prefix created by this admission is written once into its group's blocks, from the
         rows of the member whose admission created it;
      2. members of a prefix written earlier read its rows back from the shared blocks;
      3. causal attention with LSE for the computed rows ([KVS] Key techniques 2);
      4. full layer: each prompt's rows from its first unshared slot are compacted (the prefix
         stays shared); compressed layer: window score, top-k over all n tokens and compaction
         into the prompt's own blocks, which are copy-on-write replacements of shared entries
         ([KVS] Key techniques 1, 2; [PAG] How paging works).
    Returns o, lse (computed rows), scores, keep_idx, keep_offsets, kept, first (rows reused per
    prompt), cu_q, cu_k (host lists) and tables_dev.
    """
    dev = k.device
    P = cache.prefix_len
    lengths = [int(sq[2]) for sq in seqs]
    lp = [plans[sq[0]][layer] for sq in seqs]
    first = [prefix_rows_reused(cache, layer, p, n, alpha) for p, n in zip(lp, lengths)]
    cu_k = [0]
    for n in lengths:
        cu_k.append(cu_k[-1] + n)
    cu_q = [0]
    for n, f in zip(lengths, first):
        cu_q.append(cu_q[-1] + n - f)
    if k.shape[0] != cu_k[-1] or v.shape[0] != cu_k[-1] or q.shape[0] != cu_q[-1]:
        raise ValueError("q must hold each prompt's computed rows and k, v all its rows")

    def i32(x):
        return torch.tensor(x, dtype=torch.int32).to(dev)

    for s, sq in enumerate(seqs):
        if lp[s].new_prefix:
            a = cu_k[s]
            ops.kvs_compact_paged(k[a:a + P].contiguous(), v[a:a + P].contiguous(), i32([0, P]), None, None, P,
                                  k_pool, v_pool, i32([cache.prefix_blocks[layer][sq[1]]]), stream=stream)
    reusers = [s for s in range(len(seqs)) if first[s]]
    if reusers:
        ops.kvs_gather_paged(k_pool, v_pool, i32([cache.prefix_blocks[layer][seqs[s][1]] for s in reusers]),
                             i32([P] * len(reusers)), i32([cu_k[s] for s in reusers]), P, k, v, stream=stream)
    cu_k_dev = i32(cu_k)
    max_n = max(lengths)
    if reusers:
        o, lse = ops.kvs_prefill_attn_lse_chunk(q, k, v, i32(cu_q), cu_k_dev, max(cu_q[s + 1] - cu_q[s]
                                                                                    for s in range(len(seqs))),
                                                max_n, scale=scale, stream=stream)
    else:
        o, lse = ops.kvs_prefill_attn_lse(q, k, v, cu_k_dev, max_n, scale=scale, stream=stream)
    max_blocks = max(len(p.table) for p in lp)
    tbl = torch.full((len(seqs), max_blocks), -1, dtype=torch.int32)
    for s, p in enumerate(lp):
        tbl[s, :len(p.table)] = torch.tensor(p.table, dtype=torch.int32)
    tbl_dev = tbl.to(dev)
    budget = cache.budgets[layer]
    scores = keep_idx = keep_off_dev = None
    kept = [p.kept for p in lp]
    if budget is None:
        offs = [p.dst_offset for p in lp]
        segs = [(cu_k[s] + offs[s], cu_k[s + 1]) for s in range(len(seqs))]
        ks = torch.cat([k[a:b] for a, b in segs])
        vs = torch.cat([v[a:b] for a, b in segs])
        cus = [0]
        for a, b in segs:
            cus.append(cus[-1] + b - a)
        ops.kvs_compact_paged(ks, vs, i32(cus), None, None, max(b - a for a, b in segs), k_pool, v_pool, tbl_dev,
                              dst_slot_offset=i32(offs), stream=stream)
    else:
        if reusers:
            scores = ops.kvs_window_score_chunk(q, k, lse, i32(cu_q), cu_k_dev, max_n, alpha, scale=scale,
                                                stream=stream)
        else:
            scores = ops.kvs_window_score(q, k, lse, cu_k_dev, max_n, alpha, scale=scale, stream=stream)
        keep_off = [0]
        for c in kept:
            keep_off.append(keep_off[-1] + c)
        keep_off_dev = i32(keep_off)
        keep_idx = ops.kvs_topk_compact(scores, k, v, cu_k_dev, max_n, alpha, budget, keep_off_dev, k_pool, v_pool,
                                        tbl_dev, total_keep=keep_off[-1], stream=stream)
    return dict(o=o, lse=lse, scores=scores, keep_idx=keep_idx, keep_offsets=keep_off_dev, kept=kept, first=first,
                cu_q=cu_q, cu_k=cu_k, tables_dev=tbl_dev)
