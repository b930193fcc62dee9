"""Pins of the oracle's masked attention (DynamicRad, arXiv 2604.20470, §3.3 Eqs. 12-13).

* full candidate set with tau = 1 (or ratio = 1) equals dense softmax attention,
  itself checked against scipy.special.softmax;
* Eq. 13 written on a full token mask equals the kept-list form;
* closed forms: constant V, Q = 0, convex combinations, order invariance.
"""
import math

import numpy as np
import pytest
from scipy.special import softmax

from oracle import dynrad_oracle as O
import workloads


def _rand_qkv(S, D, seed):
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((S, D)), rng.standard_normal((S, D)), rng.standard_normal((S, D)))


def test_dense_attention_matches_scipy_softmax():
    q, k, v = _rand_qkv(70, 16, 0)
    ref = softmax(q @ k.T / 4.0, axis=1) @ v
    np.testing.assert_allclose(O.dense_attention(q, k, v), ref, rtol=1e-12, atol=1e-12)


@pytest.mark.parametrize("mode,ratio,tau", [("static", 1.0, 1.0), ("dynamic", 1.0, 1.0)])
def test_full_candidates_keep_all_equals_dense(mode, ratio, tau):
    w = workloads.get_workload("tiny")
    q, k, v = workloads.head_qkv(w, 0, 1)
    row_ptr, cols = O.candidate_csr(**w.radial_kwargs())
    assert row_ptr[-1] == w.num_blocks ** 2
    qb, kb = O.pool_blocks(q, w.block_size), O.pool_blocks(k, w.block_size)
    s = O.block_scores(qb, kb, row_ptr, cols)
    kept, _ = O.select_all(s, row_ptr, cols, mode, ratio=ratio, tau=tau)
    out = O.sparse_attention(q, k, v, w.block_size, kept)
    ref = softmax(q.astype(np.float64) @ k.astype(np.float64).T / math.sqrt(w.head_dim), axis=1) @ v
    np.testing.assert_allclose(out, ref, rtol=1e-10, atol=1e-12)


@pytest.mark.parametrize("S,Bs", [(256, 32), (200, 32), (300, 64)])
def test_token_mask_equals_kept_lists(S, Bs):
    rng = np.random.default_rng(S)
    q, k, v = _rand_qkv(S, 32, S)
    Sb = -(-S // Bs)
    kept = [np.sort(rng.choice(Sb, size=int(rng.integers(1, Sb + 1)), replace=False)) for _ in range(Sb)]
    a = O.sparse_attention(q, k, v, Bs, kept)
    b = O.masked_attention_dense(q, k, v, Bs, O.kept_to_block_mask(kept, Sb))
    np.testing.assert_allclose(a, b, rtol=1e-10, atol=1e-12)


def test_closed_forms():
    rng = np.random.default_rng(9)
    S, D, Bs = 190, 8, 32             # ragged: last block holds 30 tokens
    Sb = 6
    q, k, v = _rand_qkv(S, D, 9)
    kept = [np.sort(rng.choice(Sb, size=3, replace=False)) for _ in range(Sb)]
    # constant V -> constant output
    vc = np.full((S, D), 2.5)
    np.testing.assert_allclose(O.sparse_attention(q, k, vc, Bs, kept), vc, rtol=1e-13)
    # Q = 0 -> uniform weights: the mean of V over the kept valid keys
    out = O.sparse_attention(np.zeros((S, D)), k, v, Bs, kept)
    for a in range(Sb):
        keys = np.concatenate([np.arange(b * Bs, min(b * Bs + Bs, S)) for b in kept[a]])
        rows = slice(a * Bs, min(a * Bs + Bs, S))
        np.testing.assert_allclose(out[rows], np.broadcast_to(v[keys].mean(0), out[rows].shape), rtol=1e-12)
    # outputs are convex combinations of the attended V rows
    out = O.sparse_attention(q, k, v, Bs, kept)
    for a in range(Sb):
        keys = np.concatenate([np.arange(b * Bs, min(b * Bs + Bs, S)) for b in kept[a]])
        rows = slice(a * Bs, min(a * Bs + Bs, S))
        assert np.all(out[rows] <= v[keys].max(0) + 1e-12)
        assert np.all(out[rows] >= v[keys].min(0) - 1e-12)
    # the order in which kept blocks are listed does not matter
    shuffled = [rng.permutation(x) for x in kept]
    np.testing.assert_allclose(O.sparse_attention(q, k, v, Bs, shuffled), out, rtol=1e-12)


def test_tiny_workload_end_to_end_counts():
    # static r = 0.5 over 8 candidates keeps 4 per query block
    w = workloads.get_workload("tiny")
    q, k, v = workloads.head_qkv(w, 0, 0)
    row_ptr, cols = O.candidate_csr(**w.radial_kwargs())
    s = O.block_scores(O.pool_blocks(q, 32), O.pool_blocks(k, 32), row_ptr, cols)
    kept, _ = O.select_all(s, row_ptr, cols, "static", ratio=0.5)
    assert [len(x) for x in kept] == [4] * 8
    kept_d, _ = O.select_all(s, row_ptr, cols, "dynamic", tau=0.8)
    assert all(1 <= len(x) <= 8 for x in kept_d)
    # the diagonal block is the top-scored candidate of each query block here
    for a in range(8):
        lo, hi = row_ptr[a], row_ptr[a + 1]
        assert cols[lo:hi][np.argmax(s[lo:hi])] == a
