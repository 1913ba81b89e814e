"""Per-layer, per-KV-head selection of the tokens to keep (oracle; test infrastructure).

Source: [KVS] Key techniques, 2. "Attention modification": in every layer l and
head h the k_l tokens with the highest score are kept and every other KV entry
is dropped for the rest of the generation.  [KVS] System model: low-score KV
pairs are pruned while pairs with a high score *and* greater proximity are kept.

Readings:
  R5  the alpha window tokens (the nearest ones) are always kept and use alpha
      of the k_l slots; the other k_l - alpha slots go to the highest S among
      the earlier tokens i < n - alpha.
  R7  equal scores: the lower index wins, i.e. a stable sort on (-S_i, i).
  R9  k_l >= n keeps every token; the window is min(alpha, n) long.
  R10 the kept indices are returned in ascending order.
"""
from __future__ import annotations

import numpy as np


def keep_count(n: int, k_budget: int) -> int:
    """k_eff = min(k_l, n) (R9)."""
    return n if k_budget >= n else k_budget


def select_keep(S: np.ndarray, n: int, alpha: int, k_budget: int) -> np.ndarray:
    """Kept token indices (int64, ascending) of one KV head of one sequence.

    S holds the scores of tokens 0..n-1.  The candidates before the window are
    ordered by a stable sort on descending score, the first k_l - alpha are
    taken, the window is added and the union is sorted ascending.
    """
    S = np.asarray(S, dtype=np.float64)[:n]
    if k_budget >= n:
        return np.arange(n, dtype=np.int64)
    a = min(alpha, n)
    if k_budget < a:
        raise ValueError("the budget must cover the window (k_l >= alpha)")
    n_cand = n - a
    order = np.argsort(-S[:n_cand], kind="stable")      # stable: equal scores keep index order
    chosen = order[: k_budget - a]
    window = np.arange(n_cand, n)
    return np.sort(np.concatenate([chosen, window])).astype(np.int64)
