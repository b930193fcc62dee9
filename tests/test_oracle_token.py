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


# ---------------------------------------------------------------------------
# token_select_decisive: which block pairs the GPU comparison may hold to
# bit-exactness. A block pair is decisive iff no token-level decision in it can
# change when every z moves by less than the margin and every score by less
# than half the margin times (sigma + eps).
# ---------------------------------------------------------------------------

def _unsure_pairs(dec, blocks):
    return {(a, b) for a, row in zip(blocks, dec) for b in np.nonzero(~row)[0]}


def test_decisive_hand_case():
    """The hand case above (frame pair (0, 2): z(u) = (u - 1.5) / sigma with
    sigma = sqrt(47/14 - 2.25) = 1.0522, so z = -1.426, -0.475, 0.475, 1.426;
    tau_far = 0.5). B_s = 2: query block 1 holds u = 2, 3 and key blocks 4, 5
    frame 2. |z(2) - tau| = 0.0248: within a margin of 0.03, outside 0.02.
    Frame pair (2, 0) has sigma = 0, every score 0 and z = 0 < tau: its
    fallback's arg-max is a tie (top two scores equal), so every pair of
    P(2, 0) (query blocks 4, 5 against key blocks 0, 1) is unsure at any margin.
    Pairs with t <= 1 are never unsure."""
    q, k = _hand_case()
    args = (3, 4, 2, 1.0, 4.0, 100.0, 0.5)
    tie = {(4, 0), (4, 1), (5, 0), (5, 1)}
    dec = O.token_select_decisive(q, k, range(6), *args, margin=0.03, scale=1.0)
    assert _unsure_pairs(dec, range(6)) == tie | {(1, 4), (1, 5)}
    dec = O.token_select_decisive(q, k, range(6), *args, margin=0.02, scale=1.0)
    assert _unsure_pairs(dec, range(6)) == tie


def _two_frame_pair_case(top, rest, tau):
    """N_f = 3, N_t = 4, B_s = 4 (one block per frame), D = 1, scale 1:
    frame 0's queries are (1, 0.1, 0.2, 0.3) and frame 2's keys (top, rest...),
    so P(0, 2) (|u - v| <= 4: all 16 pairs) has s(u, v) = q_u k_v with the
    highest score `top` at (0, 0) and the runner-up rest[0] at (0, 1) (for
    top > rest[0] > 0.3 top). Frames 1 and 2 have zero queries."""
    q = np.zeros((12, 1))
    k = np.zeros((12, 1))
    q[0:4, 0] = [1.0, 0.1, 0.2, 0.3]
    k[8:12, 0] = [top] + list(rest)
    return [q], [k], (3, 4, 4, 1.0, 4.0, 100.0, tau)


def test_decisive_fallback_near_tie_and_max_near_tau():
    """Frame pair (0, 2) is judged as a whole: it is in doubt when no pair
    passes and the runner-up score is within margin * (sigma + eps) of the
    highest (the fallback's arg-max could move), or when the highest z lies
    within the margin of tau (whether the fallback acts could change). Block
    pair (0, 2) holds all of P(0, 2) here."""
    m = 1e-3
    # runner-up 0.9999: no pair reaches tau = 3 and the top two are 1e-4 apart
    q, k, args = _two_frame_pair_case(1.0, [1.0 - 1e-4, -1.0, -1.0], tau=3.0)
    st = O.token_frame_stats(q, k, *args[:5], 100.0, 3.0, scale=1.0)
    mu, sigma, tau, fb = st[(0, 2)]
    assert (1.0 - mu) / sigma < tau and 1e-4 <= m * sigma       # no pair passes; a near tie
    assert (0, 2) in _unsure_pairs(O.token_select_decisive(q, k, [0], *args, margin=m, scale=1.0), [0])
    # the same scores with a clear gap between the top two: decisive
    q, k, args = _two_frame_pair_case(1.0, [0.5, -1.0, -1.0], tau=3.0)
    assert not _unsure_pairs(O.token_select_decisive(q, k, [0], *args, margin=m, scale=1.0), [0])
    # the clear gap again, with tau just above the highest z: in doubt
    q, k, args = _two_frame_pair_case(1.0, [0.5, -1.0, -1.0], tau=0.0)
    mu, sigma, _, _ = O.token_frame_stats(q, k, *args[:5], 100.0, 0.0, scale=1.0)[(0, 2)]
    zmax = (1.0 - mu) / (sigma + O.EPS_NORM)
    q, k, args = _two_frame_pair_case(1.0, [0.5, -1.0, -1.0], tau=zmax + 0.5 * m)
    assert (0, 2) in _unsure_pairs(O.token_select_decisive(q, k, [0], *args, margin=m, scale=1.0), [0])
    q, k, args = _two_frame_pair_case(1.0, [0.5, -1.0, -1.0], tau=zmax + 2 * m)
    assert not _unsure_pairs(O.token_select_decisive(q, k, [0], *args, margin=m, scale=1.0), [0])


def _perturbed_selection(s, Nf, Nt, Bs, gamma, lam, stats, dz, ds, theta_c, theta_m, eps):
    """Token decisions from the definitions, written out here: for each frame
    pair (i, j) with t = |i - j|, retained iff t mod sf(t) == 0, P = {|u - v|
    <= w(t)}; t <= 1 selects all of P; t > 1 selects z + dz >= tau on P, and if
    none passes, the first (u, v) of highest s + ds on P. Aggregated to blocks
    by the oracle's pinned density control."""
    w, sf = O.distance_table(Nf, Nt, Bs, gamma, lam)
    S = Nf * Nt
    sel = np.zeros((S, S), dtype=bool)
    uu = np.arange(Nt)
    for i in range(Nf):
        for j in range(Nf):
            t = abs(i - j)
            if t % sf[t] != 0:
                continue
            P = np.abs(uu[:, None] - uu[None, :]) <= w[t]
            blk = (slice(i * Nt, (i + 1) * Nt), slice(j * Nt, (j + 1) * Nt))
            if t <= 1:
                sel[blk] = P
                continue
            mu, sigma, tau, _ = stats[(i, j)]
            z = (s[blk] - mu) / (sigma + eps) + dz[blk]
            pick = P & (z >= tau)
            if not pick.any():
                sp = np.where(P, s[blk] + ds[blk], -np.inf)
                u, v = divmod(int(np.argmax(sp)), Nt)      # first in (u, v) order
                pick[u, v] = True
            sel[blk] = pick
    S_b = -(-S // Bs)
    return [O.aggregate_block_rows(sel[a * Bs:min((a + 1) * Bs, S)], a * Bs, Bs, S, theta_c, theta_m)[0]
            for a in range(S_b)], sel


@pytest.mark.parametrize("seed,taus,theta", [(1, (0.3, 0.9), (0.0, 0.0)), (2, (-0.2, 1.4), (0.2, 0.3)),
                                             (3, (1.8, 2.6), (0.0, 0.0)), (4, (0.0, 0.0), (0.3, 0.5))])
def test_decisive_pairs_survive_bounded_perturbations(seed, taus, theta):
    """Brute force on a tiny layout (4 frames x 12 tokens, B_s = 4, D = 3,
    H_f = 2; every distance retained, windows of 4 at t = 2, 3): under random
    perturbations of every z by less than the margin and of every score by
    less than margin * (sigma + eps) / 2, and under the worst case that moves
    every z the margin's width towards its threshold, no decisive block pair
    changes. Scores here come from a plain matmul, not the oracle's code."""
    rng = np.random.default_rng(seed)
    Nf, Nt, Bs, D, gamma, lam, margin = 4, 12, 4, 3, 1.0, 2.0, 0.05
    eps = O.EPS_NORM
    q, k = _heads(rng, Nf * Nt, D)
    s = sum(qh @ kh.T for qh, kh in zip(q, k)) / 2 / math.sqrt(D)
    stats = O.token_frame_stats(q, k, Nf, Nt, Bs, gamma, lam, taus[0], taus[1], eps)
    S_b = Nf * Nt // Bs
    dec = O.token_select_decisive(q, k, range(S_b), Nf, Nt, Bs, gamma, lam, taus[0], taus[1], margin, eps)
    base = O.token_select(q, k, Nf, Nt, Bs, gamma, lam, taus[0], taus[1], theta[0], theta[1], eps)
    n_dec = sum(int(d.sum()) for d in dec)
    assert 0 < n_dec < S_b * S_b                  # both kinds occur
    # the plain re-derivation agrees with the oracle when nothing moves
    zero = np.zeros_like(s)
    blocks0, sel0 = _perturbed_selection(s, Nf, Nt, Bs, gamma, lam, stats, zero, zero, *theta, eps)
    for a, ks in enumerate(blocks0):
        np.testing.assert_array_equal(ks, base[a])
    sig = np.zeros_like(s)
    tau_of = np.zeros_like(s)
    for (i, j), (mu, sigma, tau, _) in stats.items():
        sig[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt] = sigma + eps
        tau_of[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt] = tau
    mu_of = np.zeros_like(s)
    for (i, j), (mu, sigma, tau, _) in stats.items():
        mu_of[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt] = mu
    z = np.where(sig > 0, (s - mu_of) / np.where(sig > 0, sig, 1.0), 0.0)
    trials = [(rng.uniform(-0.999, 0.999, s.shape) * margin, rng.uniform(-0.499, 0.499, s.shape) * margin * sig)
              for _ in range(40)]
    toward = -0.999 * margin * np.sign(z - tau_of)
    trials += [(toward, zero), (-toward, zero), (toward, 0.499 * margin * sig), (toward, -0.499 * margin * sig)]
    flipped = 0
    for dz, ds in trials:
        got, sel = _perturbed_selection(s, Nf, Nt, Bs, gamma, lam, stats, dz, ds, *theta, eps)
        flipped += int((sel != sel0).sum())
        for a in range(S_b):
            gm = np.zeros(S_b, dtype=bool)
            gm[got[a]] = True
            bm = np.zeros(S_b, dtype=bool)
            bm[base[a]] = True
            assert not (dec[a] & (gm != bm)).any(), (a, np.nonzero(dec[a] & (gm != bm))[0])
    assert flipped > 0                            # the perturbations do move token decisions
