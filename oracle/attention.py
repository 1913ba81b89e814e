"""Causal softmax attention, written as the two-pass definition (oracle; test infrastructure).

Source: [KVS] Key techniques, 2. "Attention modification".  The page states that
softmax over QK^T needs two passes (first the row maximum, then the sum), that
FlashAttention2 (first Fig. 7) reaches the same O in one pass by carrying O,
P and the row maximum across key blocks and dividing by l at the end, and that
the row maximum and the running sum l are computed but not returned.  The
oracle computes exactly what that one-pass kernel must equal, the plain
two-pass definition, and returns the row maximum and l as well.

Readings (the attention formula itself was lost from the page):
  R1  logits are scaled: s_ji = <q_j, k_i> / sqrt(d) unless a scale is given.
  R4  causal: row j sees keys 0..j only.
  R6  LSE is in natural-log units: LSE_j = m_j + ln(l_j).
  R8  GQA: query head h reads KV head floor(h / G), G = Hq / Hkv.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np


def _check(q, k, v):
    if q.ndim != 3 or k.ndim != 3 or v.ndim != 3:
        raise ValueError("expected q [n][Hq][d], k/v [n][Hkv][d]")
    n, hq, d = q.shape
    if k.shape != v.shape or k.shape[0] != n or k.shape[2] != d:
        raise ValueError("shape mismatch")
    if hq % k.shape[1]:
        raise ValueError("Hq must be a multiple of Hkv")
    return n, hq, k.shape[1], d


def causal_attention(q: np.ndarray, k: np.ndarray, v: np.ndarray, scale: Optional[float] = None,
                     rows: Optional[Sequence[int]] = None, row_chunk: int = 2048, q_holds_rows: bool = False):
    """One sequence: O [r][Hq][d], LSE, m, l [Hq][r] for the requested rows (default all n).

    m is the row maximum of the scaled logits and l the sum of exp(s - m);
    both are what the page says FlashAttention computes but does not return.
    Pass 1 takes the maximum, pass 2 the exponentials, their sum, the
    probabilities and O = A V.  With q_holds_rows, q[i] is the query of rows[i]
    (so long prompts need not be held whole).
    """
    if q_holds_rows:
        if rows is None or len(rows) != q.shape[0]:
            raise ValueError("q_holds_rows needs one query per requested row")
        n = k.shape[0]
        hq, d = q.shape[1], q.shape[2]
        hkv = k.shape[1]
        if hq % hkv or k.shape != v.shape or k.shape[2] != d:
            raise ValueError("shape mismatch")
        q_rows = q
    else:
        n, hq, hkv, d = _check(q, k, v)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    G = hq // hkv
    r = len(rows)
    O = np.zeros((r, hq, d))
    lse = np.zeros((hq, r))
    m_out = np.zeros((hq, r))
    l_out = np.zeros((hq, r))
    for c0 in range(0, r, row_chunk):
        rr = rows[c0:c0 + row_chunk]
        kmax = int(rr.max()) + 1                     # causal: no row needs keys beyond its own index
        visible = np.arange(kmax)[None, :] <= rr[:, None]
        qsel = q_rows[c0:c0 + len(rr)] if q_holds_rows else q[rr]
        for h in range(hq):
            g = h // G
            s = scale * (qsel[:, h, :] @ k[:kmax, g, :].T)
            s = np.where(visible, s, -np.inf)
            m = s.max(axis=1)                        # pass 1: row maximum
            e = np.exp(s - m[:, None])               # pass 2: exponentials (masked entries give 0)
            l = e.sum(axis=1)
            A = e / l[:, None]
            O[c0:c0 + len(rr), h, :] = A @ v[:kmax, g, :]
            lse[h, c0:c0 + len(rr)] = m + np.log(l)
            m_out[h, c0:c0 + len(rr)] = m
            l_out[h, c0:c0 + len(rr)] = l
    return O, lse, m_out, l_out


def attention_probs(q: np.ndarray, k: np.ndarray, scale: Optional[float] = None,
                    rows: Optional[Sequence[int]] = None) -> np.ndarray:
    """The softmax matrix A [Hq][r][n] for the requested rows (zeros above the diagonal)."""
    n, hq, d = q.shape
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    rows = np.arange(n) if rows is None else np.asarray(rows, dtype=np.int64)
    G = hq // hkv
    visible = np.arange(n)[None, :] <= rows[:, None]
    A = np.zeros((hq, len(rows), n))
    for h in range(hq):
        s = scale * (q[rows, h, :] @ k[:, h // G, :].T)
        s = np.where(visible, s, -np.inf)
        m = s.max(axis=1)
        e = np.exp(s - m[:, None])
        A[h] = e / e.sum(axis=1)[:, None]
    return A
