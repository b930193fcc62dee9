"""Pins of the oracle's candidate set (DynamicRad, arXiv 2604.20470, §3.1 Eqs. 6-7
and "Density control within blocks").

* brute force: a pure-Python loop over every token pair of tiny layouts;
* invariants: symmetry in temporal distance, the dense same-frame band,
  the diagonal, monotonicity in gamma, the lambda -> large superset;
* special cases: one frame, windows covering the frame, the tiny workload.
"""
import itertools

import numpy as np
import pytest

from oracle import dynrad_oracle as O


def brute_force_blocks(Nf, Nt, Bs, gamma, lam, theta_c, theta_m):
    """Token-level definition evaluated pair by pair, then aggregated."""
    w, sf = O.distance_table(Nf, Nt, Bs, gamma, lam)
    S = Nf * Nt
    Sb = -(-S // Bs)
    M = np.zeros((Sb, Sb), dtype=bool)
    for a in range(Sb):
        qs = list(range(a * Bs, min(a * Bs + Bs, S)))
        for b in range(Sb):
            ks = list(range(b * Bs, min(b * Bs + Bs, S)))
            active = 0
            for k in ks:
                cnt = 0
                for q in qs:
                    t = abs(q // Nt - k // Nt)
                    if t % sf[t] == 0 and abs(q % Nt - k % Nt) <= w[t]:
                        cnt += 1
                if cnt / len(qs) > theta_c:
                    active += 1
            M[a, b] = active / len(ks) > theta_m
    return M


def csr_to_dense(row_ptr, cols, Sb):
    M = np.zeros((Sb, Sb), dtype=bool)
    for a in range(Sb):
        M[a, cols[row_ptr[a]:row_ptr[a + 1]]] = True
    return M


CASES = [
    # (Nf, Nt, Bs, gamma, lam, theta_c, theta_m)
    (4, 64, 32, 1.0, 2.0, 0.0, 0.0),      # the tiny workload's layout
    (6, 40, 16, 1.0, 0.3, 0.0, 0.0),      # blocks straddle frames, sf > 1
    (9, 20, 32, 0.8, 0.1, 0.0, 0.0),      # N_t < B_s: a block spans 2-3 frames
    (8, 100, 32, 1.3, 0.25, 0.0, 0.0),    # ragged last block (800 = 25 * 32)
    (7, 90, 16, 2.0, 0.4, 0.2, 0.5),      # density control thresholds
    (5, 130, 32, 0.6, 1.0, 0.5, 0.1),
    (5, 130, 32, 0.6, 1.0, 0.03, 0.9),
    (17, 24, 64, 1.0, 0.05, 0.1, 0.2),    # B_s = 64, many frames per block
    (9, 33, 128, 1.2, 0.2, 0.1, 0.3),     # B_s = 128, a block spans up to 5 frames
]


@pytest.mark.parametrize("case", CASES)
def test_candidates_equal_brute_force(case):
    Nf, Nt, Bs = case[:3]
    Sb = O.layout(Nf, Nt, Bs)["S_b"]
    row_ptr, cols = O.candidate_csr(*case)
    np.testing.assert_array_equal(csr_to_dense(row_ptr, cols, Sb), brute_force_blocks(*case))
    for a in range(Sb):   # rows ascending, no duplicates
        r = cols[row_ptr[a]:row_ptr[a + 1]]
        assert np.all(np.diff(r) > 0)


@pytest.mark.parametrize("Nf,Nt,Bs,gamma,lam", [
    (12, 150, 32, 1.0, 4.0), (10, 77, 32, 0.7, 0.2), (9, 300, 64, 1.5, 0.1), (21, 60, 32, 1.0, 0.5)])
def test_candidate_invariants(Nf, Nt, Bs, gamma, lam):
    Sb = O.layout(Nf, Nt, Bs)["S_b"]
    S = Nf * Nt
    M = csr_to_dense(*O.candidate_csr(Nf, Nt, Bs, gamma, lam), Sb)
    # the rule depends only on |f_q - f_k| and |u_q - u_k|: symmetric
    np.testing.assert_array_equal(M, M.T)
    # diagonal, and every pair of blocks sharing a frame (t = 0 is dense)
    assert M.diagonal().all()
    frames = [set(range(a * Bs // Nt, (min(a * Bs + Bs, S) - 1) // Nt + 1)) for a in range(Sb)]
    for a, b in itertools.product(range(Sb), range(Sb)):
        if frames[a] & frames[b]:
            assert M[a, b]
    # wider windows never remove a candidate (Eq. 2 scales linearly with gamma)
    M2 = csr_to_dense(*O.candidate_csr(Nf, Nt, Bs, gamma * 1.7, lam), Sb)
    assert np.all(M2 >= M)
    # lambda large enough that sf = 1 at every distance retains every frame pair,
    # so it gives a superset of any smaller lambda
    M3 = csr_to_dense(*O.candidate_csr(Nf, Nt, Bs, gamma, 1e6), Sb)
    assert np.all(M3 >= M)


def test_adjacent_band_is_dense_when_retained():
    # sf(1) = 1 and w(1) = N_t: every token pair one frame apart is a candidate
    Nf, Nt, Bs = 6, 96, 32
    Sb = O.layout(Nf, Nt, Bs)["S_b"]
    M = csr_to_dense(*O.candidate_csr(Nf, Nt, Bs, 0.25, 4.0), Sb)
    for a in range(Sb):
        for b in range(Sb):
            fa, fb = (a * Bs) // Nt, (b * Bs) // Nt
            if abs(fa - fb) <= 1:
                assert M[a, b]


def test_special_cases():
    # one frame: everything is same-frame, so every block pair is a candidate
    row_ptr, cols = O.candidate_csr(1, 1000, 32, 1.0, 1.0)
    Sb = O.layout(1, 1000, 32)["S_b"]
    assert row_ptr[-1] == Sb * Sb
    # the tiny workload: windows (>= 32 tokens at t = 2, 3 over 64-token frames,
    # blocks of 32) reach every block, so the candidate set is full: 8 x 8
    row_ptr, cols = O.candidate_csr(4, 64, 32, 1.0, 2.0)
    assert row_ptr[-1] == 64
    # windows at least N_t everywhere and sf = 1: full set
    row_ptr, cols = O.candidate_csr(10, 50, 32, 100.0, 100.0)
    Sb = O.layout(10, 50, 32)["S_b"]
    assert row_ptr[-1] == Sb * Sb
    # theta_m = 1 can never be exceeded: nothing is a candidate
    row_ptr, cols = O.candidate_csr(4, 64, 32, 1.0, 2.0, 0.0, 1.0)
    assert row_ptr[-1] == 0


def test_window_bounds_one_frame_apart_in_distance():
    # Far-frame window check at the token level: with N_t = 64 and B_s = 16,
    # gamma = 1 at t = 2 gives w = max(16, 64/4) = 16. Query block 0 holds
    # frame-0 tokens u = 0..15; in frame 2 the keys u <= 15 + 16 = 31 pair with
    # it, i.e. key blocks 8 (u 0..15) and 9 (u 16..31), and not 10 (u 32..47).
    cols = O.candidate_row(0, 3, 64, 16, 1.0, 4.0)
    frame2 = [c for c in cols if c >= 8]
    assert frame2 == [8, 9]
