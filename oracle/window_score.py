"""Observation-window score S (oracle; test infrastructure).

Source: [KVS] Key techniques, 2. "Attention modification", the PyramidKV-style
scoring paragraphs and the modified-FlashAttention figure (second Fig. 7):
  * the last alpha prompt positions ([n - alpha, n]) are the instruction window;
  * the score of token i in a head is the sum of the softmax values A[j, i]
    over the window rows j;
  * the softmax values are rebuilt from the saved row statistics as
    p = exp(s - rowmax) / l, and a row-wise sum gives S;
  * causality and the window bound mean that only pairs (j, i) with j in the
    window and i <= j are ever visited (5000 x 256 instead of 5000 x 5000).

Readings:
  R2  the window is the last alpha rows, 0-based j in {n-alpha, ..., n-1};
      if alpha >= n every row is in the window (R9).
  R3  S_i is a plain sum, no pooling or normalisation.
  R4  A[j, i] = 0 for i > j.
  R6  exp(s - m) / l = exp(s - LSE) with LSE = m + ln l, so one saved value per
      row is enough.
  R8  GQA: the score of KV head g sums its G query heads; one score per KV head.
"""
from __future__ import annotations

import math
from typing import Optional

import numpy as np


def window_score(q: np.ndarray, k: np.ndarray, lse: np.ndarray, alpha: int,
                 scale: Optional[float] = None, window_only: bool = False) -> np.ndarray:
    """One sequence: S [Hkv][n] from the window rows of q, the keys and the saved LSE [Hq][n].

    Explicit sum in the pages' order: for every KV head g, every query head h
    of its group and every window row j, add exp(scale * q_hj . k_gi - LSE_hj)
    to S_g[i] for the keys i <= j.  With window_only, q is [a][Hq][d] and lse
    [Hq][a]: only the a = min(alpha, n) window rows (long prompts).
    """
    n = k.shape[0]
    hq, d = q.shape[1], q.shape[2]
    hkv = k.shape[1]
    if hq % hkv:
        raise ValueError("Hq must be a multiple of Hkv")
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    G = hq // hkv
    a = min(alpha, n)
    first = n - a if window_only else 0            # prompt row held at index 0 of q / lse
    if window_only and (q.shape[0] != a or lse.shape[1] != a):
        raise ValueError("window_only needs the last min(alpha, n) rows")
    S = np.zeros((hkv, n))
    for g in range(hkv):
        for h in range(g * G, (g + 1) * G):
            for j in range(n - a, n):
                s = scale * (k[:j + 1, g, :] @ q[j - first, h, :])
                S[g, :j + 1] += np.exp(s - lse[h, j - first])
    return S


def window_score_from_probs(A: np.ndarray, alpha: int, hkv: int) -> np.ndarray:
    """Second route: S [Hkv][n] summed straight from a full softmax matrix A [Hq][n][n]."""
    hq, n, _ = A.shape
    G = hq // hkv
    a = min(alpha, n)
    S = np.zeros((hkv, n))
    for h in range(hq):
        S[h // G] += A[h, n - a:, :].sum(axis=0)
    return S


def visited_pairs(n: int, alpha: int) -> int:
    """Number of (window row, key) pairs the score must visit: sum over window rows of (j + 1)."""
    a = min(alpha, n)
    return sum(j + 1 for j in range(n - a, n))
