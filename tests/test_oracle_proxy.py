"""Pins of the proxy-task objective ([DR] App. C.2 Eq. 20, C.4 Eq. 22) and of
its random-probe form."""
import math

import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O


def test_full_mask_has_zero_error_and_full_penalty():
    """Keeping every block reproduces dense attention (error 0); the sparsity is
    then 0, so Eq. 22 adds alpha * (0.8 - 0) = 8."""
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((64, 8)), rng.standard_normal((64, 8))
    kept = [np.arange(4)] * 4
    assert O.proxy_nmse_exact([q], [k], [kept], 16) == pytest.approx(0.0, abs=1e-28)
    assert O.proxy_sparsity([kept], 4) == 0.0
    assert O.proxy_loss(0.0, 0.0) == pytest.approx(8.0)


def test_hand_worked_diagonal_mask():
    """Two tokens, D = 1, q = k = (1, 0), block size 1, only the diagonal kept:
    dense rows softmax(1, 0) = (e, 1)/(e + 1) and (1/2, 1/2); sparse rows are
    the identity. Error (2/(e+1)^2 + 1/2), norm ((e^2 + 1)/(e+1)^2 + 1/2)."""
    q = np.array([[1.0], [0.0]])
    kept = [np.array([0]), np.array([1])]
    e = math.e
    num = 2.0 / (e + 1) ** 2 + 0.5
    den = (e * e + 1) / (e + 1) ** 2 + 0.5
    assert O.proxy_nmse_exact([q], [q], [kept], 1) == pytest.approx(num / den, rel=1e-14)
    assert O.proxy_sparsity([kept], 2) == 0.5
    assert O.proxy_loss(num / den, 0.5) == pytest.approx(num / den + 10 * 0.3)
    assert O.proxy_loss(0.1, 0.9) == pytest.approx(0.1)


def test_probe_estimates_the_matrix_error():
    """With Z of independent N(0, 1) entries, ||(A - A') Z||^2 / D and
    ||A Z||^2 / D estimate ||A - A'||_F^2 and ||A||_F^2 (here with 20000 probe
    columns: relative standard error well under 3%)."""
    rng = np.random.default_rng(2)
    S, D, Bs = 48, 16, 8
    q = rng.standard_normal((S, D)) * 0.8
    k = q + 0.3 * rng.standard_normal((S, D))
    kept = [np.array(sorted({a, max(0, a - 1), (a + 3) % 6})) for a in range(6)]
    d, s = O.proxy_attention_matrices(q, k, kept, Bs)
    num_exact, den_exact = ((d - s) ** 2).sum(), (d ** 2).sum()
    n_probe = 20000
    z = rng.standard_normal((S, n_probe))
    num, den = O.proxy_error_sums(q, k, z, kept, Bs)
    assert num / n_probe == pytest.approx(num_exact, rel=0.05)
    assert den / n_probe == pytest.approx(den_exact, rel=0.05)


def test_drift_generator_follows_eq20():
    """Eq. 20 keeps unit variance at every frame and gives correlation
    sqrt(1 - delta^2)^t between frames t apart; queries equal keys."""
    for delta in (0.15, 0.4):
        q, k, z = workloads.proxy_qkz(6, 16, 16, 64, 2, delta, seed=3)
        assert np.array_equal(q, k)
        X = q[0, 0].astype(np.float64).reshape(6, 256, 64)
        for f in range(6):
            assert X[f].var() == pytest.approx(1.0, abs=0.03)
        for t in (1, 3):
            corr = (X[:-t] * X[t:]).mean() / math.sqrt((X[:-t] ** 2).mean() * (X[t:] ** 2).mean())
            assert corr == pytest.approx((1 - delta * delta) ** (t / 2), abs=0.02)
        assert abs(float(np.corrcoef(z[0, 0].ravel(), q[0, 0].ravel())[0, 1])) < 0.01


def test_row_error_closed_form():
    """For one query row with dense weights a and kept key set K of mass
    m = sum_K a: the kept-block softmax is a_j / m on K, so the row's squared
    error is sum_K a_j^2 (1/m - 1)^2 + sum_{not K} a_j^2."""
    rng = np.random.default_rng(4)
    S, D, Bs = 40, 8, 8
    q, k = rng.standard_normal((S, D)), rng.standard_normal((S, D))
    kept = [np.array([0, 2, 4]), np.array([1]), np.array([0, 1, 2, 3, 4]), np.array([3]), np.array([2, 4])]
    d, s = O.proxy_attention_matrices(q, k, kept, Bs)
    logits = q @ k.T / math.sqrt(D)
    for i in range(S):
        a = np.exp(logits[i] - logits[i].max())
        a /= a.sum()
        K = np.zeros(S, dtype=bool)
        for b in kept[i // Bs]:
            K[b * Bs:(b + 1) * Bs] = True
        m = a[K].sum()
        expect = (a[K] ** 2).sum() * (1 / m - 1) ** 2 + (a[~K] ** 2).sum()
        assert ((d[i] - s[i]) ** 2).sum() == pytest.approx(expect, rel=1e-12)
