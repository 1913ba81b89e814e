"""Pins for oracle.topk: exhaustive subset enumeration on tiny inputs with exact (dyadic)
scores, ties, and the budget/window edge cases (CPU only)."""
import itertools

import numpy as np
import pytest

from oracle import select_keep, keep_count


def _brute(S, n, alpha, k):
    """Lexicographically smallest subset of the candidates with the largest score sum, plus the window."""
    a = min(alpha, n)
    if k >= n:
        return list(range(n))
    cands = range(n - a)
    best, best_sum = None, None
    for sub in itertools.combinations(cands, k - a):       # lexicographic order
        s = sum(S[i] for i in sub)
        if best_sum is None or s > best_sum:
            best, best_sum = sub, s
    return sorted(list(best) + list(range(n - a, n)))


@pytest.mark.parametrize("seed", range(40))
def test_exhaustive_small(seed):
    r = np.random.default_rng(seed)
    n = int(r.integers(2, 15))
    alpha = int(r.integers(1, n + 1))
    k = int(r.integers(min(alpha, n), n + 2))
    # dyadic scores from a few levels so sums are exact and ties are common
    S = r.integers(0, 4, size=n) / 8.0
    assert list(select_keep(S, n, alpha, k)) == _brute(S, n, alpha, k)


def test_all_equal_scores_keep_lowest_indices():
    S = np.full(100, 0.25)
    keep = select_keep(S, 100, 10, 30)
    assert list(keep) == list(range(20)) + list(range(90, 100))


def test_budget_covers_everything():
    S = np.random.default_rng(0).random(50)
    assert list(select_keep(S, 50, 8, 50)) == list(range(50))
    assert list(select_keep(S, 50, 8, 500)) == list(range(50))
    assert keep_count(50, 500) == 50 and keep_count(50, 20) == 20


def test_window_only():
    S = np.random.default_rng(1).random(40)
    assert list(select_keep(S, 40, 8, 8)) == list(range(32, 40))


def test_budget_below_window_rejected():
    with pytest.raises(ValueError):
        select_keep(np.zeros(20), 20, 8, 4)


def test_output_sorted_contains_window_and_top_scores():
    r = np.random.default_rng(2)
    n, alpha, k = 500, 32, 100
    S = r.random(n)
    keep = select_keep(S, n, alpha, k)
    assert len(keep) == k and np.all(np.diff(keep) > 0)
    assert set(range(n - alpha, n)) <= set(keep.tolist())
    chosen = [i for i in keep if i < n - alpha]
    rest = [i for i in range(n - alpha) if i not in set(chosen)]
    assert min(S[chosen]) >= max(S[rest])


def test_ties_at_the_boundary_go_to_lower_index():
    S = np.array([0.5, 0.1, 0.3, 0.3, 0.3, 0.9, 0.0, 0.0])
    # window = {6, 7}; two more slots: 0.9 (index 5), 0.5 (index 0) -> then boundary ties at 0.3 unused
    assert list(select_keep(S, 8, 2, 4)) == [0, 5, 6, 7]
    # three more slots: the first 0.3 (index 2) wins the tie
    assert list(select_keep(S, 8, 2, 5)) == [0, 2, 5, 6, 7]
