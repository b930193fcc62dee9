"""Pins of the oracle's decay-state static-ratio selection ([DR] §3.2
"Static-ratio mode", Eq. 8, Algorithm 1) and of the counter-based generator it
samples with. Each test fixes a value by a published vector, brute force, a
closed form or a statistical property of uniform sampling."""
import math
import os

import numpy as np
import pytest

from oracle import dynrad_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))


def _kat():
    rows = []
    with open(os.path.join(HERE, "golden", "philox4x32_10_kat.txt")) as fh:
        for line in fh:
            if line.strip() and not line.startswith("#"):
                rows.append([int(x, 16) for x in line.split()])
    return rows


def test_philox_known_answers():
    """The published known-answer vectors of Philox4x32-10."""
    rows = _kat()
    assert len(rows) == 3
    for c0, c1, c2, c3, k0, k1, *expect in rows:
        got = O.philox4x32_10(np.array([c0]), np.array([c1]), np.array([c2]), np.array([c3]), k0, k1)
        assert [int(x[0]) for x in got] == expect


def _brute_P(Nt, w):
    return {(u, v) for u in range(Nt) for v in range(Nt) if abs(u - v) <= w}


@pytest.mark.parametrize("Nf,Nt,Bs,gamma,lam,rn,rf", [
    (4, 64, 32, 1.0, 2.0, 0.5, 0.3),
    (6, 200, 64, 1.4, 0.7, 0.75, 0.55),     # blocks straddle frames
    (8, 256, 32, 1.4, 0.1, 0.55, 0.5),      # split stride > 1 at some distances
    (5, 100, 32, 2.0, 0.3, 0.25, 0.0),      # rho = 0 still keeps one pair
])
def test_exactly_k_pairs_of_P(Nf, Nt, Bs, gamma, lam, rn, rf):
    """Every retained frame pair with t > 1 contributes exactly
    k = max(1, floor(|P| rho)) of its own candidate pairs (|P| by brute force);
    t <= 1 contributes all of P; non-retained frame pairs nothing."""
    seed = 977 * Nf + Nt
    th = O.static_frame_thresholds(Nf, Nt, Bs, gamma, lam, rn, rf, seed)
    w, sf = O.distance_table(Nf, Nt, Bs, gamma, lam)
    sel = O.static_selected_rows(slice(0, Nf * Nt), Nf, Nt, Bs, gamma, lam, seed, th)
    for i in range(Nf):
        for j in range(Nf):
            t = abs(i - j)
            blk = sel[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt]
            picked = {(int(u), int(v)) for u, v in zip(*np.nonzero(blk))}
            if t % sf[t] != 0:
                assert not picked and (i, j) not in th
                continue
            P = _brute_P(Nt, w[t])
            assert picked <= P
            if t <= 1:
                assert picked == P
                continue
            rho = rn if O.decay_length(t, Nt, gamma) >= Bs else rf
            k = max(1, math.floor(len(P) * rho + 1e-9))
            assert th[(i, j)][:2] == (len(P), k)
            assert len(picked) == k


def test_all_pass_equals_candidate_set():
    """rho_1 = rho_2 = 1 keeps all of every P(i, j): the aggregated mask is the
    candidate CSR of the independent analytic construction (same theta)."""
    for Nf, Nt, Bs, gamma, lam, tc, tm in [(4, 64, 32, 1.0, 2.0, 0.0, 0.0), (6, 200, 64, 1.4, 0.7, 0.45, 0.7),
                                            (8, 256, 32, 1.4, 0.1, 0.3, 0.5)]:
        kept = O.static_select(Nf, Nt, Bs, gamma, lam, 1.0, 1.0, 5, tc, tm)
        rp, cols = O.candidate_csr(Nf, Nt, Bs, gamma, lam, tc, tm)
        for a, ks in enumerate(kept):
            np.testing.assert_array_equal(ks, cols[rp[a]:rp[a + 1]])


def test_near_and_far_retention():
    """Eq. 8 by decay state: N_t = 16, B_s = 2, gamma = 1: L(2) = 16/4 = 4 >= 2
    (near, rho_1); w(2) = 4, |P(0, 2)| = 16*9 - 4*5 = 124, k = 62 at rho_1 = 0.5.
    N_t = 4: L(2) = 1 < 2 (far, rho_2); w(2) = 2, |P| = 4*5 - 2*3 = 14,
    k = floor(14 * 0.3) = 4."""
    th = O.static_frame_thresholds(3, 16, 2, 1.0, 4.0, 0.5, 0.3, 11)
    assert th[(0, 2)][:2] == (124, 62) and th[(2, 0)][:2] == (124, 62)
    th = O.static_frame_thresholds(3, 4, 2, 1.0, 4.0, 0.5, 0.3, 11)
    assert th[(0, 2)][:2] == (14, 4)


def test_sample_is_uniform_over_seeds():
    """The kept pairs of P(0, 2) (14 pairs, k = 4) over 3000 seeds: each pair is
    kept with probability k/n = 2/7 and each two pairs together with
    k(k-1)/(n(n-1)) = 6/91, as for a uniformly random k-subset (6-sigma
    binomial bounds); frame pairs (0, 2) and (2, 0) draw different subsets."""
    n_seeds = 3000
    inc = np.zeros((4, 4), dtype=np.int64)
    pair_hits = {}
    same = 0
    for seed in range(n_seeds):
        th = O.static_frame_thresholds(3, 4, 2, 1.0, 4.0, 0.5, 0.3, seed)
        sel = O.static_selected_rows(slice(0, 12), 3, 4, 2, 1.0, 4.0, seed, th)
        a = sel[0:4, 8:12]
        b = sel[8:12, 0:4]
        assert a.sum() == 4 and b.sum() == 4
        inc += a
        same += int(np.array_equal(a, b))
        kept = list(zip(*np.nonzero(a)))
        for x in range(len(kept)):
            for y in range(x + 1, len(kept)):
                pair_hits[(kept[x], kept[y])] = pair_hits.get((kept[x], kept[y]), 0) + 1
    P = np.abs(np.arange(4)[:, None] - np.arange(4)[None, :]) <= 2
    p1 = 4 / 14
    sd1 = math.sqrt(n_seeds * p1 * (1 - p1))
    assert np.all(inc[~P] == 0)
    assert np.all(np.abs(inc[P] - n_seeds * p1) < 6 * sd1)
    p2 = 4 * 3 / (14 * 13)
    sd2 = math.sqrt(n_seeds * p2 * (1 - p2))
    cells = list(zip(*np.nonzero(P)))
    assert len(cells) == 14
    for x in range(14):
        for y in range(x + 1, 14):
            hits = pair_hits.get((cells[x], cells[y]), 0)
            assert abs(hits - n_seeds * p2) < 6 * sd2, (cells[x], cells[y], hits)
    # two independent 4-of-14 draws coincide with probability 1/1001
    assert same < 20


def test_seed_determines_the_mask():
    kw = dict(num_frames=6, tokens_per_frame=96, block_size=32, gamma=1.0, lam=4.0, rho_near=0.3, rho_far=0.2,
              theta_c=0.2, theta_m=0.3)
    a = O.static_select(seed=7, **kw)
    b = O.static_select(seed=7, **kw)
    c = O.static_select(seed=8, **kw)
    assert all(np.array_equal(x, y) for x, y in zip(a, b))
    assert not all(np.array_equal(x, y) for x, y in zip(a, c))


def test_near_band_always_kept():
    """rho = 0 (one pair per frame pair with t > 1): with theta = 0 every block
    pair holding a t <= 1 candidate pair is still kept (the band of Eq. 8), and
    each retained t > 1 frame pair adds exactly one token pair."""
    Nf, Nt, Bs = 6, 96, 32
    kept = O.static_select(Nf, Nt, Bs, 1.0, 4.0, 0.0, 0.0, 3)
    for a, ks in enumerate(kept):
        fa0, fa1 = a * Bs // Nt, ((a + 1) * Bs - 1) // Nt
        for b in range(Nf * Nt // Bs):
            fb0, fb1 = b * Bs // Nt, ((b + 1) * Bs - 1) // Nt
            if min(abs(fa0 - fb1), abs(fa1 - fb0), abs(fa0 - fb0), abs(fa1 - fb1)) <= 1:
                assert b in ks
    th = O.static_frame_thresholds(Nf, Nt, Bs, 1.0, 4.0, 0.0, 0.0, 3)
    sel = O.static_selected_rows(slice(0, Nf * Nt), Nf, Nt, Bs, 1.0, 4.0, 3, th)
    far = sum(int(sel[i * Nt:(i + 1) * Nt, j * Nt:(j + 1) * Nt].sum()) for (i, j) in th)
    assert far == len(th) and all(v[1] == 1 for v in th.values())
