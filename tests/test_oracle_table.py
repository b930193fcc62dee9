"""Pins of the oracle's per-distance table (DynamicRad, arXiv 2604.20470, §3.1 Eqs. 1-5).

Expected values are worked out by hand from the equations (derivations in the
comments), not produced by the oracle.
"""
import math

import numpy as np
import pytest

from oracle import dynrad_oracle as O


def test_group_index_is_floor_log2_plus_one():
    # Eq. 1 for small t, where float log2 is exact enough: B(1)=1, B(2..3)=2, B(4..7)=3.
    for t in range(1, 5000):
        assert O._group_index(t) == math.floor(math.log2(t)) + 1
    assert [O._group_index(t) for t in (1, 2, 3, 4, 7, 8, 15, 16, 31, 32)] == [1, 2, 2, 3, 3, 4, 4, 5, 5, 6]


def test_base_span_next_power_of_two():
    # Eq. 1: L0 = 2^ceil(log2 N_t).
    assert O._base_span(1560) == 2048     # 1024 < 1560 <= 2048
    assert O._base_span(3600) == 4096     # 2048 < 3600 <= 4096
    assert O._base_span(64) == 64
    assert O._base_span(65) == 128
    assert O._base_span(1) == 1


def _expect(num_frames, near, groups):
    """Build the expected w array: near = N_t for t <= 1, then group values
    for t in [2^(B-1), 2^B) (B = 2, 3, ...)."""
    w = [near, near]
    B = 2
    while len(w) < num_frames:
        for _ in range(2 ** (B - 1)):
            if len(w) < num_frames:
                w.append(groups[B - 2])
        B += 1
    return np.array(w[:num_frames])


@pytest.mark.parametrize("name,args,w_expected", [
    # 480p Wan: N_t = 30*52 = 1560, L0 = 2048, B_s = 32, gamma = 1:
    #   B=2: 2048/4 = 512; B=3: 256; B=4: 128; B=5: 64 (all >= B_s).
    ("wan480_g1", (21, 1560, 32, 1.0, 4.0), _expect(21, 1560, [512, 256, 128, 64])),
    # gamma = 0.7: 358.4 -> 358, 179.2 -> 179, 89.6 -> 90, 44.8 -> 45.
    ("wan480_g07", (21, 1560, 32, 0.7, 2.0), _expect(21, 1560, [358, 179, 90, 45])),
    # 720p Wan: N_t = 45*80 = 3600, L0 = 4096: 1024, 512, 256, 128.
    ("wan720", (21, 3600, 32, 1.0, 4.0), _expect(21, 3600, [1024, 512, 256, 128])),
    # Hunyuan 33 frames, B_s = 64: ... t = 32 has B = 6: 4096/64 = 64 = max(64, 64).
    ("hunyuan", (33, 3600, 64, 1.0, 4.0), _expect(33, 3600, [1024, 512, 256, 128, 64])),
    # tiny: N_t = 64, L0 = 64: t = 2,3 -> 64/4 = 16 < B_s -> 32.
    ("tiny", (4, 64, 32, 1.0, 2.0), np.array([64, 64, 32, 32])),
    # gamma = 2.5 at N_t = 100 (L0 = 128): t=2,3: 32*2.5 = 80; t=4..7: 16*2.5 = 40;
    # t=8..15: 8*2.5 = 20 -> max(32, 20) = 32. (lambda = 4 keeps sf = 1.)
    ("g25", (10, 100, 32, 2.5, 4.0), np.array([100, 100, 80, 80, 40, 40, 40, 40, 32, 32])),
    # N_t = 128 (L0 = 128), B_s = 16, gamma = 1.28125: t=2,3: 32*1.28125 = 41.0;
    # t=4,5: 16*1.28125 = 20.5 -> rounds half up to 21.
    ("half", (6, 128, 16, 1.28125, 4.0), np.array([128, 128, 41, 41, 21, 21])),
])
def test_window_width_hand_values(name, args, w_expected):
    w, sf = O.distance_table(*args)
    np.testing.assert_array_equal(w, w_expected)
    # with lambda >= 1 at these sizes L_split >= B_s, so sf = 1 everywhere.
    np.testing.assert_array_equal(sf, np.ones_like(sf))


def test_round_half_up_exact_tie():
    # N_t = 128, L0 = 128, B_s = 16, gamma = 1.28125: t=2: 32 * 1.28125 = 41.0;
    # gamma = 1.265625: 32 * 1.265625 = 40.5 exactly -> ties go up -> 41
    # (Python's round() would give 40).
    w, _ = O.distance_table(3, 128, 16, 1.265625, 1.0)
    assert w[2] == 41
    w, _ = O.distance_table(3, 128, 16, 1.234375, 1.0)   # 39.5 -> 40
    assert w[2] == 40


def test_split_stride_with_eps():
    # N_t = 256 (L0 = 256), B_s = 32, lambda = 0.25:
    #   t=1:     span 128, L_split 32 -> 32/32.000001 = 0.99999997 -> 0 -> sf 1
    #   t=2,3:   span 64,  L_split 16 -> 1.99999988 -> 1
    #   t=4..7:  span 32,  L_split 8  -> 3.9999995  -> 3
    #   t=8..15: span 16,  L_split 4  -> 7.999998   -> 7
    #   t=16..:  span 8,   L_split 2  -> 15.999992  -> 15
    _, sf = O.distance_table(20, 256, 32, 1.0, 0.25)
    assert list(sf) == [1, 1, 1, 1, 3, 3, 3, 3] + [7] * 8 + [15] * 4
    # without eps the exact quotients would give 2, 4, 8, 16 at t = 2, 4, 8, 16
    _, sf0 = O.distance_table(20, 256, 32, 1.0, 0.25, eps=0.0)
    assert list(sf0) == [1, 1, 2, 2, 4, 4, 4, 4] + [8] * 8 + [16] * 4


def test_split_stride_applies_to_adjacent_frames():
    # N_t = 256, B_s = 32, lambda = 0.1: t=1: L_split = 128 * 0.1 = 12.8
    #   -> 32 / 12.800001 = 2.4999998 -> sf(1) = 2, so 1 mod 2 != 0 (Eq. 6):
    #   adjacent frames are not retained under the literal rule.
    _, sf = O.distance_table(3, 256, 32, 1.0, 0.1)
    assert sf[0] == 1 and sf[1] == 2
    # t=2: span 64 -> 6.4 -> 32/6.400001 = 4.9999992 -> 4
    assert sf[2] == 4


@pytest.mark.parametrize("Nt,Bs", [(100, 32), (1560, 32), (3600, 64), (17, 32)])
def test_table_invariants(Nt, Bs):
    for gamma in (0.5, 1.0, 1.7, 3.0):
        for lam in (0.05, 0.1, 0.3, 1.0, 4.0):
            w, sf = O.distance_table(40, Nt, Bs, gamma, lam)
            assert w[0] == Nt and w[1] == Nt and sf[0] == 1
            assert np.all(sf >= 1)
            assert np.all(w[2:] >= Bs)
            assert np.all(np.diff(w[2:]) <= 0)          # windows shrink with distance
            assert np.all(np.diff(sf[1:]) >= 0)         # strides grow with distance
            w2, _ = O.distance_table(40, Nt, Bs, gamma * 1.5, lam)
            assert np.all(w2 >= w)                      # larger gamma -> wider windows (Eq. 2)
            _, sf2 = O.distance_table(40, Nt, Bs, gamma, lam * 2)
            assert np.all(sf2 <= sf)                    # larger lambda -> smaller strides (Eq. 5)
