"""Pins of the oracle's token-level dynamic-threshold selection ([DR] §3.2
Eqs. 9-11, safeguard (ii), Algorithm 1; aggregation by the density control of
§3.1). Each test fixes a value by hand arithmetic, brute force or an
independent construction."""
import math

import numpy as np
import pytest

from oracle import dynrad_oracle as O


def _heads(rng, S, D, H=2):
    return [rng.standard_normal((S, D)) for _ in range(H)], [rng.standard_normal((S, D)) for _ in range(H)]


@pytest.mark.parametrize("Nf,Nt,Bs,gamma,lam,tc,tm", [
    (4, 64, 32, 1.0, 2.0, 0.0, 0.0),
    (6, 200, 64, 1.4, 0.7, 0.45, 0.7),      # blocks straddle frames
    (8, 256, 32, 1.4, 0.1, 0.3, 0.5),       # split stride > 1 at some distances
    (5, 100, 32, 2.0, 0.3, 0.2, 0.75),
])
def test_all_pass_equals_candidate_set(Nf, Nt, Bs, gamma, lam, tc, tm):
    """tau = -inf at every distance selects all of P(i, j) (Eq. 7 on retained
    pairs): the aggregated mask must be the candidate CSR built by the
    independent analytic construction with the same (theta_c, theta_m)."""
    rng = np.random.default_rng(Nf * Nt)
    q, k = _heads(rng, Nf * Nt, 16)
    kept = O.token_select(q, k, Nf, Nt, Bs, gamma, lam, -np.inf, -np.inf, tc, tm)
    rp, cols = O.candidate_csr(Nf, Nt, Bs, gamma, lam, tc, tm)
    for a, ks in enumerate(kept):
        np.testing.assert_array_equal(ks, cols[rp[a]:rp[a + 1]])


def _hand_case():
    """N_f = 3, N_t = 4, B_s = 2, gamma = 1, lambda = 4, D = 1, scale 1.
    L0 = 4. t = 2: B(2) = 2, L(2) = 4/4 = 1 < B_s (far class), w = max(2,
    round(1)) = 2, L_split = 4, sf = max(1, floor(2/4)) = 1 (retained).
    Frame 0 queries q = 0, 1, 2, 3; frame 2 keys k = 1: s(u, v) = u on
    P(0, 2) = {|u - v| <= 2} (14 pairs: rows u = 0..3 have 3, 4, 4, 3 pairs).
    Frame 2 queries are 0: s = 0 on P(2, 0)."""
    q = np.zeros((12, 1))
    k = np.zeros((12, 1))
    q[0:4, 0] = [0, 1, 2, 3]
    k[8:12, 0] = 1.0
    k[0:4, 0] = [5, -1, 2, 7]
    return [q], [k]


def test_hand_worked_statistics_and_selection():
    q, k = _hand_case()
    st = O.token_frame_stats(q, k, 3, 4, 2, 1.0, 4.0, tau_near=100.0, tau_far=0.5, scale=1.0)
    assert set(st) == {(0, 2), (2, 0)}
    mu, sigma, tau, fb = st[(0, 2)]
    # sum s = 0*3 + 1*4 + 2*4 + 3*3 = 21; sum s^2 = 0 + 4 + 16 + 27 = 47; n = 14
    assert mu == pytest.approx(21 / 14, abs=1e-15)
    assert sigma == pytest.approx(math.sqrt(47 / 14 - (21 / 14) ** 2), abs=1e-15)
    assert tau == 0.5 and fb is None                        # far class threshold
    # z(u) = (u - 1.5) / sigma: u = 3 -> 1.426 >= 0.5; u = 2 -> 0.475 < 0.5
    sel = O.token_selected_rows(q, k, slice(0, 4), 3, 4, 2, 1.0, 4.0, st, scale=1.0)
    expect = np.zeros((4, 12), dtype=bool)
    expect[:, 0:8] = True                                  # t <= 1: frames 0 and 1 in full
    expect[3, 8 + 1:8 + 4] = True                          # u = 3, v in {1, 2, 3}
    np.testing.assert_array_equal(sel, expect)
    # P(2, 0): every score is 0, sigma = 0, z = 0 < 0.5: the fallback keeps the
    # first highest-scoring pair in (u, v) order, (0, 0)
    mu2, sigma2, tau2, fb2 = st[(2, 0)]
    assert mu2 == 0.0 and sigma2 == 0.0 and fb2 == (0, 0)
    sel2 = O.token_selected_rows(q, k, slice(8, 12), 3, 4, 2, 1.0, 4.0, st, scale=1.0)
    expect2 = np.zeros((4, 12), dtype=bool)
    expect2[:, 4:12] = True                                # frames 1, 2
    expect2[0, 0] = True                                   # the fallback pair
    np.testing.assert_array_equal(sel2, expect2)


def test_near_class_uses_tau_near():
    """N_t = 16, B_s = 2: L0 = 16, L(2) = 4 >= B_s, so t = 2 is the near class
    (Eq. 11, tau_1); with N_t = 4 (L(2) = 1) it is the far class (tau_2)."""
    rng = np.random.default_rng(3)
    for Nt, near in ((16, True), (4, False)):
        q, k = _heads(rng, 3 * Nt, 8)
        st = O.token_frame_stats(q, k, 3, Nt, 2, 1.0, 4.0, tau_near=-7.0, tau_far=7.0)
        assert st[(0, 2)][2] == (-7.0 if near else 7.0)
        assert O.decay_length(2, Nt, 1.0) == (4.0 if near else 1.0)


def test_aggregation_by_hand():
    """Query block 0 (tokens 0, 1) against keys 0..3, B_s = 2: column counts
    (2, 0, 1, 2) of 2 rows -> ratios (1, 0, 0.5, 1). theta_c = 0.5 (strict) ->
    active (T, F, F, T); each key block then has 1 of 2 active columns, 0.5."""
    sel = np.array([[1, 0, 1, 1], [1, 0, 0, 1]], dtype=bool)
    assert [list(x) for x in O.aggregate_block_rows(sel, 0, 2, 4, 0.5, 0.4)] == [[0, 1]]
    assert [list(x) for x in O.aggregate_block_rows(sel, 0, 2, 4, 0.5, 0.5)] == [[]]
    # theta_c = 0.49 also activates column 2: key block 1 has 2 of 2 active
    # columns (1 > 0.5), key block 0 still 1 of 2 (0.5, not above 0.5)
    assert [list(x) for x in O.aggregate_block_rows(sel, 0, 2, 4, 0.49, 0.5)] == [[1]]


def test_fallback_is_brute_force_argmax():
    """tau = +inf: each retained frame pair with t > 1 contributes exactly its
    highest-scoring candidate pair, found here by an explicit loop."""
    rng = np.random.default_rng(5)
    Nf, Nt, Bs = 4, 24, 8
    q, k = _heads(rng, Nf * Nt, 4)
    w, sf = O.distance_table(Nf, Nt, Bs, 1.0, 2.0)
    st = O.token_frame_stats(q, k, Nf, Nt, Bs, 1.0, 2.0, np.inf, np.inf)
    for (i, j), (mu, sigma, tau, fb) in st.items():
        best, arg = -np.inf, None
        for u in range(Nt):
            for v in range(Nt):
                if abs(u - v) <= w[abs(i - j)]:
                    s = sum(float(q[h][i * Nt + u] @ k[h][j * Nt + v]) for h in range(2)) / 2 / math.sqrt(4)
                    if s > best:
                        best, arg = s, (u, v)
        assert fb == arg
    sel = O.token_selected_rows(q, k, slice(0, Nf * Nt), Nf, Nt, Bs, 1.0, 2.0, st)
    for (i, j), (_, _, _, (u, v)) in st.items():
        blk = sel[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt]
        assert blk.sum() == 1 and blk[u, v]


def test_scale_invariance_and_monotone_threshold():
    """z is invariant to a positive rescaling of the scores (Eq. 10), so the
    selection is too; lowering both thresholds can only add pairs (theta = 0)."""
    rng = np.random.default_rng(9)
    Nf, Nt, Bs = 6, 64, 16
    q, k = _heads(rng, Nf * Nt, 16)
    base = O.token_select(q, k, Nf, Nt, Bs, 1.0, 2.0, 0.3, 1.2)
    scaled = O.token_select([3.0 * x for x in q], k, Nf, Nt, Bs, 1.0, 2.0, 0.3, 1.2)
    for a, b in zip(base, scaled):
        np.testing.assert_array_equal(a, b)
    lower = O.token_select(q, k, Nf, Nt, Bs, 1.0, 2.0, -0.5, 0.4)
    for a, b in zip(base, lower):
        assert set(a.tolist()) <= set(b.tolist())


def test_rows_subset_matches_full():
    rng = np.random.default_rng(11)
    Nf, Nt, Bs = 5, 48, 16
    q, k = _heads(rng, Nf * Nt, 8)
    full = O.token_select(q, k, Nf, Nt, Bs, 1.2, 0.5, -0.5, 1.5, 0.3, 0.4)
    part = O.token_select_rows(q, k, [3, 7, 14], Nf, Nt, Bs, 1.2, 0.5, -0.5, 1.5, 0.3, 0.4)
    for a, ks in zip([3, 7, 14], part):
        np.testing.assert_array_equal(ks, full[a])
