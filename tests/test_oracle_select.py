"""Pins of the oracle's block scoring and dual-mode selection.

Static-ratio keeps exactly max(1, ceil(r * n)) candidates (checked in exact
rational arithmetic on the decimal ratio); dynamic-threshold keeps the minimal
descending-score prefix whose softmax mass reaches tau (checked by exhaustive
subset search on short rows and by the mass inequalities on long ones).
"""
import itertools
import math
from fractions import Fraction

import numpy as np
import pytest
from scipy.special import softmax

from oracle import dynrad_oracle as O


@pytest.mark.parametrize("ratio", ["0.1", "0.15", "0.2", "0.5", "0.3", "0.75", "1.0", "0.05"])
def test_static_count_is_ceil_ratio_times_n(ratio):
    r = Fraction(ratio)
    for n in range(1, 6000):
        expect = max(1, math.ceil(r * n))
        assert O.static_count(n, float(ratio)) == expect, (ratio, n)


def test_static_select_brute_force():
    rng = np.random.default_rng(1)
    for n in range(1, 11):
        cols = np.sort(rng.choice(1000, size=n, replace=False))
        s = rng.standard_normal(n)
        for ratio in (0.1, 0.3, 0.5, 0.9, 1.0):
            k = O.static_count(n, ratio)
            kept = O.select_static(s, cols, ratio)
            assert len(kept) == k
            best = max(itertools.combinations(range(n), k), key=lambda idx: s[list(idx)].sum())
            np.testing.assert_array_equal(kept, np.sort(cols[list(best)]))


def test_static_select_long_rows_and_ties():
    rng = np.random.default_rng(2)
    cols = np.sort(rng.choice(5000, size=900, replace=False))
    s = rng.standard_normal(900)
    kept = O.select_static(s, cols, 0.15)
    assert len(kept) == math.ceil(Fraction("0.15") * 900)
    in_kept = np.isin(cols, kept)
    assert s[in_kept].min() >= s[~in_kept].max()
    # all scores equal: ties go to the lowest key-block indices
    kept = O.select_static(np.zeros(10), np.arange(10) * 3, 0.3)
    np.testing.assert_array_equal(kept, [0, 3, 6])


def exhaustive_dynamic(s, tau):
    """Smallest subset (ties: largest mass) whose softmax mass reaches tau."""
    p = softmax(s)
    n = len(s)
    for k in range(1, n + 1):
        best = max(itertools.combinations(range(n), k), key=lambda idx: p[list(idx)].sum())
        if p[list(best)].sum() >= tau:
            return sorted(best)
    return list(range(n))


def test_dynamic_select_exhaustive():
    rng = np.random.default_rng(3)
    for trial in range(200):
        n = int(rng.integers(1, 11))
        s = rng.standard_normal(n) * float(rng.choice([0.05, 0.5, 2.0]))
        cols = np.arange(n) * 7 + 3
        for tau in (0.05, 0.3, 0.5, 0.8, 0.95):
            kept = O.select_dynamic(s, cols, tau)
            idx = exhaustive_dynamic(s, tau)
            assert len(kept) == len(idx), (trial, tau)
            np.testing.assert_array_equal(kept, cols[idx])


def test_dynamic_mass_inequalities_long_rows():
    rng = np.random.default_rng(4)
    for _ in range(20):
        n = int(rng.integers(200, 1100))
        s = rng.standard_normal(n) * 0.05
        cols = np.sort(rng.choice(3000, size=n, replace=False))
        p = softmax(s)
        prev = None
        for tau in (0.1, 0.5, 0.8, 0.85, 0.99):
            kept = O.select_dynamic(s, cols, tau)
            m = np.isin(cols, kept)
            assert p[m].sum() >= tau
            # dropping the lowest-scored kept block falls below tau
            weakest = np.argmin(np.where(m, s, np.inf))
            assert p[m].sum() - p[weakest] < tau
            # every kept score beats every dropped score
            if (~m).any():
                assert s[m].min() >= s[~m].max()
            if prev is not None:
                assert set(prev) <= set(kept)   # nested in tau
            prev = kept


def test_dynamic_edge_cases():
    s = np.array([0.3, -1.0, 2.0, 0.1])
    cols = np.array([1, 4, 9, 12])
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 1.0), cols)        # tau = 1 keeps all
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 1e-12), [9])       # fallback: top one
    # equal scores: softmax is uniform; tau = 0.5 over 4 needs exactly 2 (lowest indices)
    np.testing.assert_array_equal(O.select_dynamic(np.zeros(4), cols, 0.5), [1, 4])
    # worked by hand: p = softmax([ln 6, ln 3, ln 1]) = [0.6, 0.3, 0.1]
    s = np.log(np.array([6.0, 3.0, 1.0]))
    cols = np.array([0, 1, 2])
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 0.6), [0])
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 0.61), [0, 1])
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 0.9), [0, 1])
    np.testing.assert_array_equal(O.select_dynamic(s, cols, 0.91), [0, 1, 2])


def test_margins():
    s = np.array([0.5, 0.4, 0.1, 0.0])
    cols = np.arange(4)
    # static r = 0.5 keeps 2: margin s_2 - s_3 = 0.3
    assert math.isclose(O.selection_margin(s, cols, "static", ratio=0.5), 0.3)
    assert O.selection_margin(s, cols, "static", ratio=1.0) == math.inf
    # dynamic: p = [6, 3, 1] / 10 (hand), tau = 0.8 keeps 2; cum = 0.6, 0.9
    s = np.log(np.array([6.0, 3.0, 1.0]))
    m = O.selection_margin(s, np.arange(3), "dynamic", tau=0.8)
    assert math.isclose(m, min(0.9 - 0.8, 0.8 - 0.6, math.log(3.0) - 0.0), rel_tol=1e-12)


def test_pooling_and_scores():
    rng = np.random.default_rng(5)
    S, D, Bs = 100, 16, 32           # ragged last block of 4 rows
    x = rng.standard_normal((S, D))
    xb = O.pool_blocks(x, Bs)
    assert xb.shape == (4, D)
    # sum of (valid count * mean) equals the plain column sum
    counts = np.array([32, 32, 32, 4])
    np.testing.assert_allclose((counts[:, None] * xb).sum(0), x.sum(0), rtol=1e-12, atol=1e-12)
    # constant blocks pool to their constant; padding never enters the mean
    c = np.repeat(np.arange(4.0), [32, 32, 32, 4])[:, None] * np.ones((1, D))
    np.testing.assert_array_equal(O.pool_blocks(c, Bs), np.arange(4.0)[:, None] * np.ones((1, D)))
    # scores: the dense product Qbar Kbar^T / sqrt(D) read at the candidate entries
    qb, kb = rng.standard_normal((6, D)), rng.standard_normal((6, D))
    row_ptr = np.array([0, 2, 2, 5, 6, 6, 9])
    cols = np.array([0, 5, 1, 2, 3, 4, 0, 2, 5])
    s = O.block_scores(qb, kb, row_ptr, cols)
    full = qb @ kb.T / math.sqrt(D)
    rows = np.repeat(np.arange(6), np.diff(row_ptr))
    np.testing.assert_allclose(s, full[rows, cols], rtol=1e-13)
    # fused heads average the per-head scores (Eq. 19)
    qb2, kb2 = rng.standard_normal((6, D)), rng.standard_normal((6, D))
    f = O.fused_scores([qb, qb2], [kb, kb2], row_ptr, cols)
    np.testing.assert_allclose(f, 0.5 * (full + qb2 @ kb2.T / math.sqrt(D))[rows, cols], rtol=1e-13)
