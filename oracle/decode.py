"""Attention of one new token over its cached keys and values (oracle; test infrastructure).

Source: [PAG] "How paging works": the attention kernel reads a request's keys and
values back through its block table, block by block; the cache itself holds
every earlier token.  [KVS] Key techniques 2, last paragraph: PagedAttention does
the decode-side work over the (compressed) cache.

The oracle takes the cache already gathered (``paged.gather_rows``) and computes
the plain two-pass softmax for the single query row: every cached token is in
the past, so there is no mask.

Readings: R1 (scale 1/sqrt(d)), R6 (natural-log LSE), R8 (KV head = h // G),
R14 (the new token is written to slot L-1 first and attends to itself).
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def decode_attention(q: np.ndarray, k_ctx: np.ndarray, v_ctx: np.ndarray, scale: Optional[float] = None):
    """q [Hq][d], k_ctx/v_ctx [L][Hkv][d] -> (o [Hq][d], lse [Hq])."""
    hq, d = q.shape
    L, hkv, _ = k_ctx.shape
    if L == 0:
        raise ValueError("empty context")
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = hq // hkv
    o = np.zeros((hq, d))
    lse = np.zeros(hq)
    for h in range(hq):
        s = scale * (k_ctx[:, h // G, :] @ q[h])
        m = s.max()
        e = np.exp(s - m)
        l = e.sum()
        o[h] = (e / l) @ v_ctx[:, h // G, :]
        lse[h] = m + math.log(l)
    return o, lse
