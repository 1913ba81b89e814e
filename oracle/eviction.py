"""Decode-time scoring and eviction in a compressed layer (oracle; test infrastructure).

Source: [KVS] Key techniques 1, "step preparation": the layers after the third use a
sliding-window strategy that automatically replaces the KV entries with the lowest
scores, under a fixed per-layer budget.  [KVS] Key techniques 2, last paragraph:
PagedAttention does work like FlashAttention's, with the shared goal of the score S.

Readings (plainest ones the pages support):
  R20  decode rows extend the window rows of the prefill score: a cached token's score
       starts at its prefill S (0 for tokens appended during decode), and every decode
       step adds its softmax probability from each of the G query heads of its KV head.
  R21  the cache of a compressed layer holds at most `cap` = k_l tokens per KV head.
       While it has room the new token is appended (slot n_filled, the same in every
       head); once full, each KV head replaces its lowest-score token among those older
       than the alpha most recent positions (the window stays, as at prefill), ties going
       to the older position.  The new token starts at score 0.
  R14  (as for plain decode) the new token is written first and attends to itself; the
       step's probabilities are added after the attention.

State of one sequence in one layer, per KV head g (numpy arrays, fp64):
  k, v    [Hkv][cap][d]   slot contents (only the first n_filled slots are live)
  score   [Hkv][cap]      accumulated score
  pos     [Hkv][cap]      prompt-local position of the token in each slot (-1 = empty)
  n       int             filled slots
"""
from __future__ import annotations

import math
from dataclasses import dataclass
from typing import Optional

import numpy as np


@dataclass
class SlotCache:
    k: np.ndarray
    v: np.ndarray
    score: np.ndarray
    pos: np.ndarray
    n: int
    cap: int


def init_cache(k_rows: np.ndarray, v_rows: np.ndarray, scores: np.ndarray, keep: np.ndarray, cap: int) -> SlotCache:
    """Cache after compaction: head g holds tokens keep[g] (ascending) with their prefill scores.

    k_rows, v_rows [n][Hkv][d] (the prompt), scores [Hkv][n] (the window score S),
    keep [Hkv][k_eff] (the kept indices).
    """
    hkv, k_eff = keep.shape
    d = k_rows.shape[2]
    if k_eff > cap:
        raise ValueError("more kept tokens than slots")
    c = SlotCache(np.zeros((hkv, cap, d)), np.zeros((hkv, cap, d)), np.zeros((hkv, cap)),
                  np.full((hkv, cap), -1, dtype=np.int64), k_eff, cap)
    for g in range(hkv):
        c.k[g, :k_eff] = k_rows[keep[g], g]
        c.v[g, :k_eff] = v_rows[keep[g], g]
        c.score[g, :k_eff] = scores[g, keep[g]]
        c.pos[g, :k_eff] = keep[g]
    return c


def select_slot(score: np.ndarray, pos: np.ndarray, n: int, cap: int, new_pos: int, alpha: int) -> int:
    """R21: the slot of one KV head that receives the token at position new_pos."""
    if n < cap:
        return n
    best = None
    for t in range(cap):
        if pos[t] >= new_pos - alpha:          # one of the alpha most recent: kept
            continue
        key = (score[t], pos[t])
        if best is None or key < best[0]:
            best = (key, t)
    if best is None:
        raise ValueError("no slot may be replaced (cap <= alpha)")
    return best[1]


def decode_step(c: SlotCache, q: np.ndarray, new_k: np.ndarray, new_v: np.ndarray, new_pos: int, alpha: int,
                scale: Optional[float] = None, dst: Optional[np.ndarray] = None):
    """One decode step of one sequence: q [Hq][d], new_k/new_v [Hkv][d].

    Returns (o [Hq][d], lse [Hq], dst [Hkv]); the cache is updated in place.  A caller that
    has already decided the slots (a GPU run being followed step by step) passes dst.
    """
    hq, d = q.shape
    hkv = c.k.shape[0]
    G = hq // hkv
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if dst is None:
        dst = np.array([select_slot(c.score[g], c.pos[g], c.n, c.cap, new_pos, alpha) for g in range(hkv)])
    for g in range(hkv):
        c.k[g, dst[g]] = new_k[g]
        c.v[g, dst[g]] = new_v[g]
        c.score[g, dst[g]] = 0.0
        c.pos[g, dst[g]] = new_pos
    c.n = min(c.n + 1, c.cap)
    o = np.zeros((hq, d))
    lse = np.zeros(hq)
    gain = np.zeros((hkv, c.n))
    for h in range(hq):
        g = h // G
        s = scale * (c.k[g, :c.n] @ q[h])
        m = s.max()
        l = np.exp(s - m).sum()
        lse[h] = m + math.log(l)
        p = np.exp(s - lse[h])
        o[h] = p @ c.v[g, :c.n]
        gain[g] += p
    c.score[:, :c.n] += gain                    # after the attention (R20, R14)
    return o, lse, dst
