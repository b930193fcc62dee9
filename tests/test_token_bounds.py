"""The bound with which the token selector's decision pass (B_s = 32) fixes a
key column as active or inactive without its logits ([DR] §3.1 "Density
control within blocks": a key token is active when the share of its selected
query tokens exceeds theta_c; §3.2 Eqs. 10-11 select a pair when its score
reaches the frame pair's threshold).

Cantelli's one-sided inequality on a column's n values bounds how many of them
reach a threshold T from the values' mean and population variance. The
kernel takes both from float32 sums formed as the statistics pass forms them
(each lane adds its 16 rows in order, sums of squares by fused multiply-add,
the two lanes of a column added last), widened by the float32 rounding
bounds. This test restates that decision in NumPy and checks, on many columns
of adversarial values, that a fixed column never contradicts the exact count,
and that the rounding bounds it assumes hold. CPU only; it checks the rule,
not the kernel (the GPU tests compare the kernel's kept lists with the
oracle)."""
import math

import numpy as np
import pytest

U = 2.0 ** -24
F32 = np.float32


def _row_halves(n_rows=32):
    """Row indices held by the two lanes of a key column, in summation order
    (lane half h holds rows 8 * (i // 4) + 4 * h + i % 4, i = 0..15)."""
    return [[8 * (i // 4) + 4 * h + (i % 4) for i in range(16)] for h in (0, 1)]


def _fma32(a, b, c):
    """float32 fused multiply-add: a * b + c rounded once (a * b of two float32
    values is exact in float64; the sum is exact for the magnitudes here)."""
    return (a.astype(np.float64) * b.astype(np.float64) + c.astype(np.float64)).astype(F32)


def column_sums(vals, inwin):
    """float32 (sum, sum of squares) of each column's in-window values, formed
    as the kernel forms them. vals: [m, 32] float32; inwin: [m, 32] bool."""
    m = vals.shape[0]
    halves = []
    for rows in _row_halves():
        ts = np.zeros(m, F32)
        tq = np.zeros(m, F32)
        for r in rows:
            x = vals[:, r]
            w = inwin[:, r]
            ts = np.where(w, (ts + x).astype(F32), ts)
            tq = np.where(w, _fma32(x, x, tq), tq)
        halves.append((ts, tq))
    cs = (halves[0][0] + halves[1][0]).astype(F32)
    cq = (halves[0][1] + halves[1][1]).astype(F32)
    return cs, cq


def decide(cs, cq, n, T, min_c, widen=True):
    """The decision pass's rule per column (threshold T[i]): (active, inactive)
    fixed. widen=False drops the rounding bounds (a planted mistake)."""
    act = np.zeros(len(cs), bool)
    inact = np.zeros(len(cs), bool)
    for i in range(len(cs)):
        ni = int(n[i])
        if ni == 0:
            act[i] = 0 >= min_c
            inact[i] = not act[i]
            continue
        nn = float(ni)
        S1, Q = float(cs[i]), float(cq[i])
        Qhi = Q * (1.0 + 20.0 * U) if widen else Q
        e1s = 20.0 * U * float(np.sqrt(np.float32(nn * Qhi))) * (1.0 + 1e-6) if widen else 0.0
        sa = max(0.0, abs(S1) - e1s)
        M = max(0.0, nn * Qhi - sa * sa)          # >= n^2 x the population variance
        A = nn * float(T[i]) - S1
        # Cantelli, multiplied through by n^2 (var + d^2)
        if A - e1s > 0.0:
            dn = A - e1s
            inact[i] = nn * M * (1.0 + 1e-12) < min_c * (M + dn * dn)
        elif -A - e1s > 0.0:
            dn = -A - e1s
            act[i] = nn * dn * dn * (1.0 - 1e-12) > (min_c - 1) * (M + dn * dn)
    return act, inact


def _columns(kind, m, rng):
    if kind == "gauss":
        return rng.standard_normal((m, 32)).astype(F32) * F32(11.3)
    if kind == "outlier":
        v = rng.standard_normal((m, 32)).astype(F32) * F32(3.0)
        v[np.arange(m), rng.integers(0, 32, m)] += F32(150.0)
        return v
    if kind == "two_point":
        return np.where(rng.random((m, 32)) < rng.random((m, 1)), F32(-20.0), F32(30.0)).astype(F32)
    if kind == "constant":
        return np.repeat(rng.standard_normal((m, 1)).astype(F32) * F32(10.0), 32, axis=1)
    if kind == "offset":
        # large mean, tiny spread: the mean's square dwarfs the variance
        return (F32(1000.0) + rng.standard_normal((m, 32)).astype(F32) * F32(0.01)).astype(F32)
    if kind == "cancel":
        s = np.where(rng.random((m, 32)) < 0.5, F32(-1.0), F32(1.0))
        return (s * (F32(500.0) + rng.random((m, 32)).astype(F32))).astype(F32)
    raise ValueError(kind)


KINDS = ["gauss", "outlier", "two_point", "constant", "offset", "cancel"]


@pytest.mark.parametrize("kind", KINDS)
@pytest.mark.parametrize("cut", [False, True])
def test_fixed_columns_agree_with_exact_counts(kind, cut):
    rng = np.random.default_rng([KINDS.index(kind), int(cut)])
    m = 3000
    vals = _columns(kind, m, rng)
    if cut:
        # a window edge: each column keeps a contiguous run of rows
        lo = rng.integers(0, 32, m)
        hi = np.minimum(31, lo + rng.integers(0, 32, m))
        r = np.arange(32)[None, :]
        inwin = (r >= lo[:, None]) & (r <= hi[:, None])
    else:
        inwin = np.ones((m, 32), bool)
    n = inwin.sum(axis=1)
    cs, cq = column_sums(vals, inwin)
    # thresholds around the columns' own means, some far, some near
    mean = np.where(n > 0, (vals * inwin).sum(axis=1) / np.maximum(n, 1), 0.0)
    spread = np.sqrt(np.maximum((vals.astype(np.float64) ** 2 * inwin).sum(axis=1) / np.maximum(n, 1) - mean ** 2, 0))
    T = (mean + rng.uniform(-4.0, 4.0, m) * (spread + 1e-3)).astype(F32)
    fixed = 0
    for min_c in (1, 8, 15, 24, 32):
        act, inact = decide(cs, cq, n, T.astype(np.float64), min_c)
        count = ((vals >= T[:, None]) & inwin).sum(axis=1)
        assert not np.any(act & (count < min_c)), "a column fixed active has fewer selected values"
        assert not np.any(inact & (count >= min_c)), "a column fixed inactive has enough selected values"
        assert not np.any(act & inact)
        fixed += int(act.sum() + inact.sum())
    if kind in ("gauss", "two_point", "constant"):
        assert fixed > 0, "the rule fixes nothing on ordinary columns"


@pytest.mark.parametrize("kind", KINDS)
def test_float32_sums_within_the_assumed_bounds(kind):
    """|cs - sum x| <= 20 u sqrt(n Qhi) and sum x^2 <= cq (1 + 20 u), the
    widening the rule applies."""
    rng = np.random.default_rng(100 + KINDS.index(kind))
    m = 4000
    vals = _columns(kind, m, rng)
    inwin = np.ones((m, 32), bool)
    cs, cq = column_sums(vals, inwin)
    v64 = vals.astype(np.float64)
    exact_s = v64.sum(axis=1)
    exact_q = (v64 ** 2).sum(axis=1)
    qhi = cq.astype(np.float64) * (1.0 + 20.0 * U)
    assert np.all(exact_q <= qhi * (1 + 1e-15))
    assert np.all(np.abs(cs.astype(np.float64) - exact_s) <= 20.0 * U * np.sqrt(32.0 * qhi))


def test_cantelli_is_tight_enough_for_the_papers_thresholds():
    """On unit-variance columns a threshold 2 deviations above the mean (the
    far threshold of Table 2 "mid") leaves at most n / 5 of 32 values, below
    the 15 of theta_c = 0.45; 1.5 deviations below (the near threshold) leaves
    at least 32 - 32 / 3.25 = 22.2: both fixed."""
    rng = np.random.default_rng(7)
    x = rng.standard_normal((200, 32))
    x = ((x - x.mean(axis=1, keepdims=True)) / x.std(axis=1, keepdims=True)).astype(F32)
    n = np.full(200, 32)
    cs, cq = column_sums(x, np.ones((200, 32), bool))
    act, inact = decide(cs, cq, n, 2.0 * np.ones(200), 15)
    assert inact.all() and not act.any()
    act, inact = decide(cs, cq, n, -1.5 * np.ones(200), 15)
    assert act.all() and not inact.any()


def test_the_rounding_widening_is_needed():
    """Without the float32 rounding bounds the rule fixes columns wrongly when
    the mean's square dwarfs the variance: the cancellation in sum x^2 - (sum
    x)^2 / n leaves a variance below the true one."""
    rng = np.random.default_rng(5)
    m = 20000
    vals = _columns("offset", m, rng)
    n = np.full(m, 32)
    cs, cq = column_sums(vals, np.ones((m, 32), bool))
    v64 = vals.astype(np.float64)
    T = (v64.mean(axis=1) + rng.uniform(-4.0, 4.0, m) * (v64.std(axis=1) + 1e-3)).astype(F32)
    count = (vals >= T[:, None]).sum(axis=1)
    wrong = {}
    for widen in (False, True):
        act, inact = decide(cs, cq, n, T.astype(np.float64), 15, widen=widen)
        wrong[widen] = int(np.sum(act & (count < 15)) + np.sum(inact & (count >= 15)))
    assert wrong[False] > 0 and wrong[True] == 0
