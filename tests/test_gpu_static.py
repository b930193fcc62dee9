"""GPU parity of dr_static_select (the decay-state static-ratio selector,
[DR] §3.2 Eq. 8, Algorithm 1) against the oracle: integer work, so the kept
lists must match bit for bit on every (b, h), and the per-frame-pair sample
cut (k-th smallest Philox word, position cut among its ties) must equal the
oracle's k-th smallest sort key."""
import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

STATE_WORDS = 12   # uint32 fields per frame pair at the start of the workspace


def _run(Nf, Nt, Bs, gamma, lam, tc, tm, rn, rf, seed, batch=1, heads=1):
    cand = G.dr().build_candidates(G.dr().radial_cfg(Nf, Nt, Bs, gamma, lam, tc, tm))
    kept = G.dr().static_select(cand, rn, rf, seed, batch=batch, heads=heads)
    return cand, kept


def _state(cand, rn, rf, seed):
    """Run once more with a caller-owned workspace and return the per-frame-pair
    state words [Nf * Nf, 12]."""
    import ctypes
    import torch
    from block_sparse_attention_candidates_amd import _lib as L
    n = ctypes.c_size_t(0)
    assert L.lib().dr_static_select_workspace(ctypes.byref(cand.cfg), cand.nnz, ctypes.byref(n)) == 0
    ws = torch.zeros(n.value, dtype=torch.uint8, device="cuda")
    G.dr().static_select(cand, rn, rf, seed, workspace=ws)
    torch.cuda.synchronize()
    nfp = cand.cfg.num_frames ** 2
    return ws[:nfp * STATE_WORDS * 4].cpu().numpy().view(np.uint32).reshape(nfp, STATE_WORDS)


def _compare_rows(cand, kept, Nf, Nt, Bs, gamma, lam, tc, tm, rn, rf, seed, blocks=None, bh_count=1, label=""):
    rp, cols = G.host_csr(cand)
    Sb = cand.num_blocks
    blocks = list(range(Sb)) if blocks is None else blocks
    ora = O.static_select_rows(blocks, Nf, Nt, Bs, gamma, lam, rn, rf, seed, tc, tm)
    for bh in range(bh_count):
        lists = G.kept_lists(kept, rp, cand.nnz, Sb, bh)
        for a, o in zip(blocks, ora):
            np.testing.assert_array_equal(lists[a], o, err_msg=f"{label} (b, h) #{bh} row {a}")
    kept_total = sum(len(o) for o in ora)
    G.log(f"   {label}: {len(blocks)} rows equal, {kept_total} kept of {sum(rp[a + 1] - rp[a] for a in blocks)}"
          f" candidates")


@pytest.mark.parametrize("rho", [(0.5, 0.3), (1.0, 1.0), (0.0, 0.0)])
@pytest.mark.parametrize("theta", [(0.0, 0.0), (0.2, 0.3)])
@pytest.mark.parametrize("seed", [7, (1 << 40) + 3])
def test_static_tiny(rho, theta, seed):
    G.log(f"[static] tiny rho={rho} theta={theta} seed={seed}")
    w = workloads.get_workload("tiny")
    args = (w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam, theta[0], theta[1], rho[0], rho[1], seed)
    cand, kept = _run(*args)
    _compare_rows(cand, kept, *args, label="tiny")


@pytest.mark.parametrize("preset", ["low", "mid", "high"])
def test_static_presets_small_video(preset):
    """8 frames of 16x16 tokens, B_s = 32, with [DR] Table 2's static presets."""
    G.log(f"[static] small video, preset {preset}")
    pr = workloads.STATIC_PRESETS[preset]
    args = (8, 256, 32, pr["gamma"], pr["lam"], pr["theta_c"], pr["theta_m"], pr["rho_near"], pr["rho_far"], 11)
    cand, kept = _run(*args)
    _compare_rows(cand, kept, *args, label=f"small/{preset}")


def test_static_straddling_bs64_batch2_heads3():
    """6 frames of 200 tokens (64-token blocks straddle frames), written for
    2 x 3 (b, h): every copy equals the oracle's mask."""
    G.log("[static] B_s = 64 straddling, batch 2 x heads 3")
    args = (6, 200, 64, 1.4, 0.7, 0.2, 0.3, 0.3, 0.2, 123456789)
    cand, kept = _run(*args, batch=2, heads=3)
    _compare_rows(cand, kept, *args, bh_count=6, label="bs64")


@pytest.mark.parametrize("case", [(6, 200, 128, 1.4, 0.7, 0.2, 0.3, 0.3, 0.2, 77),
                                  (9, 33, 128, 1.2, 0.2, 0.1, 0.3, 0.5, 0.4, 78)])
def test_static_block_size_128(case):
    """B_s = 128, incl. N_t = 33 where a block spans up to 5 frames."""
    G.log(f"[static] B_s = 128 {case}")
    cand, kept = _run(*case)
    _compare_rows(cand, kept, *case, label="bs128")


def test_static_split_stride():
    """lambda = 0.1: sf(t) > 1 drops whole frame distances (Eq. 6)."""
    G.log("[static] split stride > 1")
    args = (8, 256, 32, 1.4, 0.1, 0.1, 0.1, 0.4, 0.3, 5)
    cand, kept = _run(*args)
    _compare_rows(cand, kept, *args, label="sf>1")


def _check_cuts(state, Nf, Nt, Bs, gamma, lam, rn, rf, seed, pairs):
    w, sf = O.distance_table(Nf, Nt, Bs, gamma, lam)
    for (i, j) in pairs:
        t = abs(i - j)
        keys = O.static_frame_sorted_keys(i, j, Nt, w[t], seed)
        k = O.static_pair_count(len(keys), O.static_rho(t, Nt, Bs, gamma, rn, rf))
        K = int(keys[k - 1])
        T, pos = K >> 32, K & 0xFFFFFFFF
        tie_after = k < len(keys) and int(keys[k]) >> 32 == T
        st = state[i * Nf + j]
        assert st[0] == 1 and st[2] == len(keys) and st[3] == k, (i, j, st[:4])
        assert st[6] == T, (i, j, hex(st[6]), hex(T))
        assert st[9] == (pos if tie_after else 0xFFFFFFFF), (i, j, st[9], pos, tie_after)
        G.log(f"   ({i}, {j}): |P| {len(keys)}, k {k}, word cut {T:#010x}, tie after the cut: {tie_after}")


def test_static_full_size_cuts_and_rows():
    """wan13b_480p shape under the Table 2 'mid' static preset: the sample cut
    of every frame pair of two query frames, and the kept lists of sampled
    query blocks of those frames."""
    G.log("[static] wan13b_480p + static mid: cuts and sampled rows")
    w, (rn, rf) = workloads.static_workload("wan13b_480p", "mid")
    Nf, Nt, Bs = w.num_frames, w.tokens_per_frame, w.block_size
    seed = 2024
    cand, kept = _run(Nf, Nt, Bs, w.gamma, w.lam, w.theta_c, w.theta_m, rn, rf, seed)
    state = _state(cand, rn, rf, seed)
    frames = [3, 17]
    _, sf = O.distance_table(Nf, Nt, Bs, w.gamma, w.lam)
    pairs = [(i, j) for i in frames for j in range(Nf) if abs(i - j) > 1 and abs(i - j) % sf[abs(i - j)] == 0]
    _check_cuts(state, Nf, Nt, Bs, w.gamma, w.lam, rn, rf, seed, pairs[::4])
    blocks = [a for a in G.sample_blocks(w.num_blocks, 400, seed=9)
              if a * Bs // Nt in frames and ((a + 1) * Bs - 1) // Nt in frames][:12]
    _compare_rows(cand, kept, Nf, Nt, Bs, w.gamma, w.lam, w.theta_c, w.theta_m, rn, rf, seed, blocks=blocks,
                  label="wan13b_480p+static-mid")


def test_static_tied_word_position_cut():
    """3 frames of 60x60 tokens, gamma = 4 (P(0, 2) is all N_t^2 = 12,960,000
    pairs), rho = 0.5, seed 1060: the k-th smallest word of P(0, 2) is shared
    with a pair of larger position, so the cut needs the position passes."""
    G.log("[static] tied word at the cut")
    args = (3, 3600, 32, 4.0, 4.0, 0.0, 0.0, 0.5, 0.5, 1060)
    cand, _ = _run(*args)
    state = _state(cand, 0.5, 0.5, 1060)
    assert state[0 * 3 + 2][8] == 1   # the position passes ran for (0, 2)
    _check_cuts(state, 3, 3600, 32, 4.0, 4.0, 0.5, 0.5, 1060, [(0, 2), (2, 0)])
