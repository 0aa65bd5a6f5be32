"""Pins of the oracle's composite score and top-N selection.

CONF-KV explainer, Methodology, token ranking and eviction: tokens are ranked
by a composite of EMA attention mass and recency within the chosen budget; a
hard protected window P keeps the newest tokens.  Significance and claims: the
method is a no-op while the context stays under its budget.
"""
import itertools

import numpy as np
import pytest

from oracle import composite_scores, select_keep

F32 = np.float32


def _beats(a, b, s, pos):
    """Total order used for ranking: higher score first, newer position on ties."""
    return (s[a] > s[b]) or (s[a] == s[b] and pos[a] > pos[b])


@pytest.mark.parametrize("seed", range(25))
def test_brute_force_unique_subset(seed):
    rng = np.random.default_rng(seed)
    n = int(rng.integers(3, 13))
    t = int(rng.integers(n - 1, 3 * n))
    pos = np.sort(rng.choice(np.arange(t), size=n - 1, replace=False))
    pos = np.append(pos, t)                                  # the newest token is cached
    P = int(rng.integers(1, 4))
    N = int(rng.integers(max(P, 1), n))                      # n > N: eviction happens
    if rng.random() < 0.5:                                   # many ties
        s = rng.integers(0, 3, n).astype(F32) / F32(4)
    else:
        s = rng.random(n).astype(F32)
    keep = select_keep(s, pos, t, P, N)
    prot = pos > t - P
    cand = [i for i in range(n) if not prot[i]]
    K = N - int(prot.sum())
    valid = []
    for sub in itertools.combinations(cand, K):
        rest = [i for i in cand if i not in sub]
        if all(_beats(a, b, s, pos) for a in sub for b in rest):
            valid.append(set(sub))
    assert len(valid) == 1                                   # exactly one correct keep set
    want = np.zeros(n, bool)
    want[list(valid[0])] = True
    want |= prot
    assert np.array_equal(keep, want)
    assert keep.sum() == N


def test_no_op_at_or_under_budget():
    pos = np.arange(10)
    s = np.random.default_rng(0).random(10).astype(F32)
    assert select_keep(s, pos, 9, 3, 10).all()
    assert select_keep(s, pos, 9, 3, 50).all()
    assert select_keep(s, pos, 9, 3, 9).sum() == 9


def test_protected_window_survives_low_scores():
    pos = np.arange(100)
    s = np.ones(100, F32)
    s[-8:] = 0                       # the newest 8 score worst, yet P = 8 keeps them
    keep = select_keep(s, pos, 99, 8, 20)
    assert keep[-8:].all() and keep.sum() == 20


def test_ties_keep_newer():
    pos = np.array([3, 5, 9, 11, 20])
    s = np.array([0.5, 0.5, 0.5, 0.5, 0.0], F32)
    keep = select_keep(s, pos, 20, 1, 3)
    assert list(pos[keep]) == [9, 11, 20]


def test_composite_score_values():
    e = np.array([0.0, 0.02, 0.04, 0.01], F32)
    pos = np.array([0, 10, 30, 40])
    s = composite_scores(e, pos, 40, 0.7, 0.3)
    # the newest token with the largest mass: 0.7f + 0.3f rounds to exactly 1.0f
    assert composite_scores(np.array([1.0], F32), np.array([40]), 40, 0.7, 0.3)[0] == F32(1.0)
    assert s[0] == F32(0.0)
    # e/e_max = 0.5, pos/t = 0.25: two fp32 products then an fp32 add
    want = F32(F32(0.7) * F32(F32(0.02) / F32(0.04))) + F32(F32(0.3) * F32(F32(10) / F32(40)))
    assert s[1] == want
    assert s.dtype == F32


def test_composite_score_monotone_and_bounded():
    rng = np.random.default_rng(3)
    e = rng.random(500).astype(F32) * F32(1e-3)
    pos = np.arange(500)
    s = composite_scores(e, pos, 499, 0.7, 0.3)
    assert np.all((s >= 0) & (s <= 1))
    i, j = 10, 11
    e2 = e.copy()
    e2[i] = e2[j] = F32(5e-4)
    s2 = composite_scores(e2, pos, 499, 0.7, 0.3)
    assert s2[j] >= s2[i]                                    # same mass: newer ranks higher
    assert composite_scores(np.zeros(4, F32), np.arange(4), 3, 0.7, 0.3)[3] == F32(0.3)
    assert composite_scores(np.ones(1, F32), np.array([0]), 0, 0.7, 0.3)[0] == F32(1.0)
