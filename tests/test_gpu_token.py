"""GPU parity of dr_token_select (the token-level dynamic-threshold selector,
[DR] §3.2 Eqs. 9-11, Algorithm 1) against the oracle.

A block pair is compared bit-exactly where the oracle's decision is decisive:
every t > 1 candidate pair of it lies more than MARGIN (in z units) from its
threshold and no fallback it could receive is in doubt. Elsewhere the GPU
decision only has to stay inside the candidate set. Every head carries the
same mask.
"""
import dataclasses
import math

import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

MARGIN = 1e-3


def _device(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _run_and_compare(qb, kb, Nf, Nt, Bs, gamma, lam, tc, tm, tau_near, tau_far, Hf, blocks=None, label=""):
    """qb, kb: uint16 bf16 patterns [B, H, S, D]. Returns (decisive, compared) counts."""
    B, H, S, D = qb.shape
    q, k = _device(qb), _device(kb)
    cand = G.dr().build_candidates(G.dr().radial_cfg(Nf, Nt, Bs, gamma, lam, tc, tm))
    kept = G.dr().token_select(q, k, cand, tau_near, tau_far, fused_heads=Hf)
    rp, cols = G.host_csr(cand)
    Sb = cand.num_blocks
    blocks = list(range(Sb)) if blocks is None else blocks
    dec_total = cmp_total = 0
    for b in range(B):
        qh = [_f64(qb[b, h]) for h in range(Hf)]
        kh = [_f64(kb[b, h]) for h in range(Hf)]
        top2 = {}
        stats = O.token_frame_stats(qh, kh, Nf, Nt, Bs, gamma, lam, tau_near, tau_far, top2=top2)
        ora = O.token_select_rows(qh, kh, blocks, Nf, Nt, Bs, gamma, lam, tau_near, tau_far, tc, tm, stats=stats)
        dec = O.token_select_decisive(qh, kh, blocks, Nf, Nt, Bs, gamma, lam, tau_near, tau_far, MARGIN,
                                      stats=stats, top2=top2)
        lists = [G.kept_lists(kept, rp, cand.nnz, Sb, b * H + h) for h in range(H)]
        for h in range(1, H):
            for a in blocks:
                np.testing.assert_array_equal(lists[h][a], lists[0][a], err_msg=f"{label} head {h} row {a}")
        for a, o, d in zip(blocks, ora, dec):
            g = lists[0][a]
            row = cols[rp[a]:rp[a + 1]]
            assert np.isin(g, row).all(), f"{label} b{b} row {a}: kept block outside the candidate set"
            gm = np.zeros(Sb, dtype=bool)
            gm[g] = True
            om = np.zeros(Sb, dtype=bool)
            om[o] = True
            bad = np.nonzero(d & (gm != om))[0]
            assert len(bad) == 0, f"{label} b{b} row {a}: decisive blocks differ at {bad[:8]} (gpu {gm[bad[:8]]})"
            dec_total += int(d[row].sum())
            cmp_total += len(row)
    G.log(f"   {label}: {dec_total}/{cmp_total} candidate block pairs decisive, all equal")
    return dec_total, cmp_total


def _random_bits(rng, shape):
    return workloads.bf16_bits(rng.standard_normal(shape).astype(np.float32))


@pytest.mark.parametrize("taus", [(-1.5, 2.0), (0.5, 1.0), (-math.inf, -math.inf), (math.inf, math.inf)])
@pytest.mark.parametrize("theta", [(0.0, 0.0), (0.45, 0.7)])
def test_token_select_tiny(taus, theta):
    """The tiny workload (4 frames of 8x8 tokens, B_s = 32, D = 64, 2 heads)."""
    G.log(f"[token] tiny taus={taus} theta={theta}")
    w = workloads.get_workload("tiny")
    qb, kb, _ = G.host_qkv("tiny")
    d, c = _run_and_compare(qb, kb, w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam, theta[0],
                            theta[1], taus[0], taus[1], 2, label="tiny")
    # the oracle marks at most 5 of 64 (resp. 2 of 52) candidate pairs unsure here
    assert d >= 0.9 * c


@pytest.mark.parametrize("preset", ["low", "mid", "high"])
def test_token_select_presets_small_video(preset):
    """8 frames of 16x16 tokens (AR(1) field, shift 1), D = 128, 4 heads,
    B_s = 32, with [DR] Table 2's dynamic presets."""
    G.log(f"[token] small video, preset {preset}")
    pr = workloads.TOKEN_PRESETS[preset]
    w = dataclasses.replace(workloads.get_workload("wan13b_480p"), name="tok_small", heads=4, num_frames=8,
                            frame_h=16, frame_w=16, seed=21)
    qb, kb, _ = workloads.qkv(w, as_bits=True)
    d, c = _run_and_compare(qb, kb, w.num_frames, w.tokens_per_frame, 32, pr["gamma"], pr["lam"], pr["theta_c"],
                            pr["theta_m"], pr["tau_near"], pr["tau_far"], 2, label=f"small/{preset}")
    assert d > 0.9 * c


def test_token_select_straddling_blocks_bs64_hf1_batch2():
    """6 frames of 200 tokens (64-token blocks straddle frames), D = 64,
    3 heads, batch 2, one fused head, theta = (0.3, 0.5)."""
    G.log("[token] B_s = 64 straddling, H_f = 1, batch 2")
    rng = np.random.default_rng(17)
    qb = _random_bits(rng, (2, 3, 1200, 64))
    kb = _random_bits(rng, (2, 3, 1200, 64))
    d, c = _run_and_compare(qb, kb, 6, 200, 64, 1.2, 0.5, 0.3, 0.5, -0.5, 1.5, 1, label="bs64")
    # 4096 token pairs per block pair of iid scores: 331 of 540 are decisive
    assert d >= 0.5 * c


def test_token_select_straddling_blocks_bs32_hf1_batch2():
    """B_s = 32 (the decision pass and the open-entry kernel): 6 frames of 200
    tokens, so query and key blocks straddle frames, D = 64, 3 heads, batch 2
    (the column sums and open marks of each batch element apart), one fused
    head, theta = (0.3, 0.5)."""
    G.log("[token] B_s = 32 straddling, H_f = 1, batch 2")
    rng = np.random.default_rng(19)
    qb = _random_bits(rng, (2, 3, 1200, 64))
    kb = _random_bits(rng, (2, 3, 1200, 64))
    d, c = _run_and_compare(qb, kb, 6, 200, 32, 1.2, 0.5, 0.3, 0.5, -0.5, 1.5, 1, label="bs32")
    assert d >= 0.75 * c                          # 1839 of 2248 are decisive


def test_token_select_block_size_128():
    """B_s = 128: 6 frames of 200 tokens (blocks span up to 2 frames), D = 128,
    2 heads fused, theta = (0.2, 0.4)."""
    G.log("[token] B_s = 128")
    rng = np.random.default_rng(29)
    qb = _random_bits(rng, (1, 2, 1200, 128))
    kb = _random_bits(rng, (1, 2, 1200, 128))
    d, c = _run_and_compare(qb, kb, 6, 200, 128, 1.2, 0.5, 0.2, 0.4, -0.5, 1.5, 2, label="bs128")
    assert d >= 0.6 * c                           # 53 of 72 are decisive


def test_token_select_full_size_sampled():
    """wan13b_480p shape (21 frames x 1560 tokens, 12 heads) with the Table 2
    'mid' preset: oracle statistics over every frame pair, decisions compared
    on sampled query blocks."""
    G.log("[token] wan13b_480p + mid, sampled rows")
    w, (tn, tf) = workloads.token_workload("wan13b_480p", "mid")
    qb, kb, _ = G.host_qkv("wan13b_480p")
    blocks = G.sample_blocks(w.num_blocks, 24, seed=3)
    d, c = _run_and_compare(qb[:, :2], kb[:, :2], w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam,
                            w.theta_c, w.theta_m, tn, tf, 2, blocks=blocks, label="wan13b_480p+mid")
    # a block pair holds ~1000 token pairs at this size, so one within MARGIN of
    # its threshold is common; the share compared must still be most of them
    assert d > 0.75 * c


def test_token_select_deterministic_and_band():
    """Two calls give identical masks; every candidate block pair whose token
    pairs all have t <= 1 is kept (tau = -inf there)."""
    import torch
    G.log("[token] determinism and near band, wan14b_720p + mid")
    w, (tn, tf) = workloads.token_workload("wan14b_720p", "mid")
    q, k, _ = G.device_qkv("wan14b_720p")
    q, k = q[:, :2].contiguous(), k[:, :2].contiguous()
    cand = G.dr().build_candidates(G.dr().radial_cfg(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma,
                                                     w.lam, w.theta_c, w.theta_m))
    k1 = G.dr().token_select(q, k, cand, tn, tf)
    k2 = G.dr().token_select(q, k, cand, tn, tf)
    rp, cols = G.host_csr(cand)
    Sb, S, Nt, Bs = cand.num_blocks, w.seq_len, w.tokens_per_frame, w.block_size
    # (only the first kept_cnt entries of a row are written: compare the lists)
    assert torch.equal(k1.kept_cnt, k2.kept_cnt)
    lists = G.kept_lists(k1, rp, cand.nnz, Sb, 0)
    for a, (x, y) in enumerate(zip(lists, G.kept_lists(k2, rp, cand.nnz, Sb, 0))):
        np.testing.assert_array_equal(x, y, err_msg=f"row {a}")
    band = 0
    for a in range(Sb):
        fa0, fa1 = a * Bs // Nt, (min(S, (a + 1) * Bs) - 1) // Nt
        kept = set(lists[a].tolist())
        for b in cols[rp[a]:rp[a + 1]]:
            fb0, fb1 = b * Bs // Nt, (min(S, (b + 1) * Bs) - 1) // Nt
            if max(abs(fa0 - fb1), abs(fa1 - fb0)) <= 1:
                band += 1
                assert int(b) in kept, f"row {a}: near-band block {b} dropped"
    density = sum(len(x) for x in lists) / Sb ** 2
    G.log(f"   {band} near-band block pairs kept; mask density {density:.3f} "
          f"(candidates {cand.nnz / Sb ** 2:.3f})")


def _kept_by_row(kept, cand, B, H):
    """Kept lists of every (b, h, row) as compact host arrays (entries past a
    row's count are not part of the result)."""
    import torch
    cnt = kept.kept_cnt.view(B * H, cand.num_blocks).cpu().numpy()
    col = kept.kept_col.view(B * H, cand.nnz).cpu().numpy()
    rp = cand.row_ptr.cpu().numpy()
    out = []
    for bh in range(B * H):
        for a in range(cand.num_blocks):
            out.append(col[bh, rp[a]:rp[a] + cnt[bh, a]].copy())
    return out


@pytest.mark.parametrize("case", ["wan13b_480p_mid", "bs64_mid"])
def test_decision_pass_equals_ring_mark(case, monkeypatch):
    """At B_s <= 64 the mark pass is the decision kernel (flags fixed from the
    statistics pass's column sums by exact counts or Cantelli bounds) plus the
    open-entry kernel; DR_TOKEN_RING_MARK=1 selects the ring mark pass, which
    computes every tile. The kept lists must be equal on every row: the full
    wan13b_480p shape under Table 2 "mid" (B_s = 32), and a B_s = 64 layout
    whose blocks straddle frames (9 frames of 40x42 tokens)."""
    import torch
    G.log(f"[token] decision pass vs ring mark: {case}")
    if case == "wan13b_480p_mid":
        w, (tn, tf) = workloads.token_workload("wan13b_480p", "mid")
        q, k, _ = G.device_qkv("wan13b_480p")
        bs = w.block_size
    else:
        pr = workloads.TOKEN_PRESETS["mid"]
        w = dataclasses.replace(workloads.get_workload("hunyuan_720p"), name="tok_bs64", heads=3, num_frames=9,
                                frame_h=40, frame_w=42, seed=23, gamma=pr["gamma"], lam=pr["lam"],
                                theta_c=pr["theta_c"], theta_m=pr["theta_m"])
        tn, tf = pr["tau_near"], pr["tau_far"]
        qb, kb, _ = workloads.qkv(w, as_bits=True)
        q, k = _device(qb), _device(kb)
        bs = 64
    cand = G.dr().build_candidates(G.dr().radial_cfg(w.num_frames, w.tokens_per_frame, bs, w.gamma, w.lam,
                                                     w.theta_c, w.theta_m))
    B, H = q.shape[0], q.shape[1]
    monkeypatch.delenv("DR_TOKEN_RING_MARK", raising=False)
    fast = G.dr().token_select(q, k, cand, tn, tf, fused_heads=2)
    torch.cuda.synchronize()
    monkeypatch.setenv("DR_TOKEN_RING_MARK", "1")
    # the library reads the C environment at each call: the setting must be visible there
    import ctypes
    libc = ctypes.CDLL(None)
    libc.getenv.restype = ctypes.c_char_p
    assert libc.getenv(b"DR_TOKEN_RING_MARK") == b"1"
    ring = G.dr().token_select(q, k, cand, tn, tf, fused_heads=2)
    torch.cuda.synchronize()
    monkeypatch.delenv("DR_TOKEN_RING_MARK")
    assert torch.equal(fast.kept_cnt, ring.kept_cnt), "kept counts differ"
    lf, lr = _kept_by_row(fast, cand, B, H), _kept_by_row(ring, cand, B, H)
    for i, (x, y) in enumerate(zip(lf, lr)):
        np.testing.assert_array_equal(x, y, err_msg=f"{case}: row {i % cand.num_blocks} of (b, h) {i // cand.num_blocks}")
    G.log(f"   {case}: {int(fast.kept_cnt.sum())} kept block pairs, equal")
