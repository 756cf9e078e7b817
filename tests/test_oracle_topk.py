"""Pins for the oracle's top-k selection (CPU only).

The oracle sorts (score desc, index asc) with qsort and keeps the head.  The
pins use other routes to the same answer: a hand-worked example, a brute
force over every subset of a tiny candidate list (the selection is the only
subset of size min(k, n) whose every member precedes every non-member), and
closed forms for all-equal / monotone lists, signed zeros, infinities and
the k >= n / n = 0 cases.
"""
import itertools
import json
import os

import numpy as np
import pytest

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _precedes(s, a, c):
    return s[a] > s[c] or (s[a] == s[c] and a < c)


def _brute_force(s, n, k):
    """The unique subset of size min(k, n) that is closed upward in the order."""
    size = min(k, n)
    found = []
    for sub in itertools.combinations(range(n), size):
        inside = set(sub)
        if all(_precedes(s, a, c) for a in sub for c in range(n) if c not in inside):
            found.append(sub)
    assert len(found) == 1
    return list(found[0]) + [-1] * (k - size)


def test_golden_worked_example(oracle):
    g = json.load(open(os.path.join(GOLDEN, "topk_worked.json")))
    s = np.array([float(v) for v in g["scores"]], dtype=np.float32)
    assert np.signbit(s[4]) and not np.signbit(s[5])
    for case in g["cases"]:
        got = oracle.topk(s[None], [case["n_cand"]], case["k"])[0]
        assert got.tolist() == case["expected"], case["why"]


@pytest.mark.parametrize("n", [1, 2, 3, 4, 5, 6])
def test_exhaustive_tie_patterns(oracle, n):
    # every pattern over three levels (plenty of ties), every k
    pats = np.array(list(itertools.product([0.0, 1.0, 2.0], repeat=n)), dtype=np.float32)
    for k in range(1, n + 2):
        got = oracle.topk(pats, [n] * len(pats), k)
        for p, row in zip(pats, got):
            assert row.tolist() == _brute_force(p, n, k)


def test_random_small_lists_with_signed_zeros_and_infinities(oracle):
    rng = np.random.default_rng(0)
    levels = np.array([-np.inf, -1.0, -0.0, 0.0, 1.0, np.inf], dtype=np.float32)
    for _ in range(300):
        n = int(rng.integers(0, 9))
        s = np.zeros(9, dtype=np.float32)
        s[:n] = rng.choice(levels, size=n)
        k = int(rng.integers(1, 11))
        got = oracle.topk(s[None], [n], k)[0]
        assert got.tolist() == _brute_force(s, n, k)


def test_closed_forms(oracle):
    n, k = 1000, 64
    eq = np.full(n, 0.5, dtype=np.float32)
    dec = -np.arange(n, dtype=np.float32)
    inc = np.arange(n, dtype=np.float32)
    got = oracle.topk(np.stack([eq, dec, inc]), [n, n, n], k)
    assert got[0].tolist() == list(range(k))
    assert got[1].tolist() == list(range(k))
    assert got[2].tolist() == list(range(n - k, n))


def test_selection_is_closed_upward_at_scale(oracle):
    rng = np.random.default_rng(1)
    n, k = 20000, 512
    s = rng.standard_normal(n).astype(np.float32)
    dup = rng.integers(0, n, size=n // 100)
    s[rng.integers(0, n, size=n // 100)] = s[dup]  # 1% exact duplicates
    got = oracle.topk(s[None], [n], k)[0]
    assert np.all(np.diff(got) > 0) and len(got) == k
    chosen = np.zeros(n, bool)
    chosen[got] = True
    lo = s[chosen].min()
    assert s[~chosen].max() <= lo
    # at the boundary value, the chosen ones are the lowest indices
    tie_in = np.nonzero(chosen & (s == lo))[0]
    tie_out = np.nonzero(~chosen & (s == lo))[0]
    if len(tie_out):
        assert tie_in.max() < tie_out.min()
