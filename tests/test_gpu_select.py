"""GPU parity of dr_score_select against the oracle.

Full-size launches (every head of each workload); the oracle checks every
head at the small sizes and a head sample {0, H/2, H-1, periodic heads} at
the large ones. Scores within 2e-5 of the float64 oracle; kept lists
bit-exact wherever the oracle's margin at the cut exceeds 1e-5, and valid
selections (count / mass) on the remaining rows.
"""
import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu

CASES = [
    ("tiny", "static", 0.5, 1.0), ("tiny", "dynamic", 1.0, 0.8),
    ("wan13b_480p", "static", 0.2, 1.0), ("wan13b_480p", "dynamic", 1.0, 0.8),
    ("wan14b_480p", "dynamic", 1.0, 0.8), ("wan14b_480p", "static", 0.2, 1.0),
    ("wan14b_720p", "static", 0.15, 1.0), ("wan14b_720p", "dynamic", 1.0, 0.8),
    ("hunyuan_720p", "dynamic", 1.0, 0.85), ("hunyuan_720p", "static", 0.1, 1.0),
]


def _static_exact_on_gpu_scores(gpu_lists, gpu_scores, row_ptr, cols, ratio):
    """The static cut is pure order statistics: on the kernel's own float32
    scores the oracle's selection (score descending, ties to the lower key
    index, k = max(1, ceil(r n))) must give the same kept lists, bit for bit,
    on every row."""
    s = gpu_scores.astype(np.float64)
    for a, g in enumerate(gpu_lists):
        lo, hi = row_ptr[a], row_ptr[a + 1]
        o = O.select_static(s[lo:hi], cols[lo:hi], ratio)
        assert np.array_equal(g, o), f"row {a}: gpu {g[:8]}.. != selection on its own scores {o[:8]}.."


@pytest.mark.parametrize("name,mode,ratio,tau", CASES)
def test_score_select_parity(name, mode, ratio, tau):
    G.log(f"[select] {name} {mode} r={ratio} tau={tau}")
    w = workloads.get_workload(name)
    q, k, _ = G.device_qkv(name)
    cand = G.candidates(name)
    rp, cols = G.host_csr(cand)
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau, return_scores=True)
    scores = kept.scores.cpu().numpy().reshape(w.batch * w.heads, cand.nnz)
    heads = range(w.heads) if w.heads * cand.nnz <= 6e6 else G.sampled_heads(w)
    tot_dec = tot_nondec = 0
    for h in heads:
        s, ora, margins = G.oracle_head_selection(name, 0, h, mode, ratio, tau, rp, cols)
        np.testing.assert_allclose(scores[h], s, rtol=1e-5, atol=G.SCORE_ATOL, err_msg=f"head {h} scores")
        gl = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h)
        d, nd = G.check_selection(gl, ora, margins, s, rp, cols, mode, ratio, tau)
        tot_dec += d
        tot_nondec += nd
        if mode == "static":
            _static_exact_on_gpu_scores(gl, scores[h], rp, cols, ratio)
    G.log(f"   decisive rows {tot_dec}, within-margin rows {tot_nondec}")
    assert tot_dec > 0.5 * (tot_dec + tot_nondec)


def test_fused_heads_share_one_mask():
    # score_heads = 2: scores are the mean over heads 0 and 1 ([DR] Eq. 19) and
    # every head receives the same kept lists.
    name = "wan13b_480p"
    G.log("[select] fused heads")
    w = workloads.get_workload(name)
    q, k, _ = G.device_qkv(name)
    cand = G.candidates(name)
    rp, cols = G.host_csr(cand)
    kept = G.dr().score_select(q, k, cand, mode="dynamic", tau=0.8, score_heads=2, return_scores=True)
    qk = [G.head_f64(name, 0, h)[:2] for h in (0, 1)]
    s = O.fused_scores([O.pool_blocks(x[0], 32) for x in qk], [O.pool_blocks(x[1], 32) for x in qk], rp, cols)
    np.testing.assert_allclose(kept.scores.cpu().numpy(), s, rtol=1e-5, atol=G.SCORE_ATOL)
    ora, margins = O.select_all(s, rp, cols, "dynamic", tau=0.8)
    gl0 = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, 0)
    G.check_selection(gl0, ora, margins, s, rp, cols, "dynamic", 1.0, 0.8)
    for h in range(1, w.heads):
        gl = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h)
        assert all(np.array_equal(x, y) for x, y in zip(gl, gl0))


def test_select_edge_cases_and_determinism():
    import torch
    G.log("[select] edge cases")
    name = "wan13b_480p"
    q, k, _ = G.device_qkv(name)
    cand = G.candidates(name)
    rp, _ = G.host_csr(cand)
    n = np.diff(rp)
    # ratio = 1 and tau = 1 keep every candidate
    for kw in (dict(mode="static", ratio=1.0), dict(mode="dynamic", tau=1.0)):
        kept = G.dr().score_select(q, k, cand, **kw)
        cnt = kept.kept_cnt.cpu().numpy().reshape(12, -1)
        assert (cnt == n[None, :]).all()
    # a tiny tau keeps exactly the top-scored block (the fallback)
    kept = G.dr().score_select(q, k, cand, mode="dynamic", tau=1e-9)
    assert (kept.kept_cnt.cpu().numpy() == 1).all()
    # a tiny ratio keeps exactly one
    kept = G.dr().score_select(q, k, cand, mode="static", ratio=1e-6)
    assert (kept.kept_cnt.cpu().numpy() == 1).all()
    # bitwise reproducible
    a = G.dr().score_select(q, k, cand, mode="dynamic", tau=0.8, return_scores=True)
    b = G.dr().score_select(q, k, cand, mode="dynamic", tau=0.8, return_scores=True)
    assert torch.equal(a.kept_cnt, b.kept_cnt) and torch.equal(a.scores, b.scores)
    ca, cb = a.kept_cnt.cpu().numpy(), b.kept_cnt.cpu().numpy()
    for bh in range(12):
        la = G.kept_lists(a, rp, cand.nnz, cand.num_blocks, bh)
        lb = G.kept_lists(b, rp, cand.nnz, cand.num_blocks, bh)
        assert all(np.array_equal(x, y) for x, y in zip(la, lb))


@pytest.mark.parametrize("mode,ratio,tau", [("static", 0.3, 1.0), ("dynamic", 1.0, 0.8)])
def test_score_select_block_size_128(mode, ratio, tau):
    """B_s = 128 ([DR] Table 4): 10 frames of 300 tokens (ragged last block),
    3 heads, D = 128, random bf16 Q/K, every head against the oracle."""
    import torch
    G.log(f"[select] B_s = 128 {mode}")
    rng = np.random.default_rng(128)
    H, S, D, Bs = 3, 3000, 128, 128
    bits = workloads.bf16_bits(rng.standard_normal((2, 1, H, S, D)).astype(np.float32))
    q, k = (torch.from_numpy(np.ascontiguousarray(bits[i])).view(torch.bfloat16).cuda() for i in range(2))
    f64 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cand = G.dr().build_candidates(G.dr().radial_cfg(10, 300, Bs, 1.0, 0.5))
    rp, cols = G.host_csr(cand)
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau, return_scores=True)
    scores = kept.scores.cpu().numpy().reshape(H, cand.nnz)
    for h in range(H):
        s = O.block_scores(O.pool_blocks(f64[0, 0, h], Bs), O.pool_blocks(f64[1, 0, h], Bs), rp, cols)
        ora, margins = O.select_all(s, rp, cols, mode, ratio=ratio, tau=tau)
        np.testing.assert_allclose(scores[h], s, rtol=1e-5, atol=G.SCORE_ATOL, err_msg=f"head {h} scores")
        gl = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h)
        G.check_selection(gl, ora, margins, s, rp, cols, mode, ratio, tau)


@pytest.mark.parametrize("mode,ratio,tau", [("static", 0.2, 1.0), ("dynamic", 1.0, 0.8)])
def test_score_select_long_rows(mode, ratio, tau):
    """4 frames of 24,000 tokens, B_s = 32 (S_b = 3000), gamma = 1: rows of
    about 2000 to 2760 candidates, so one call selects short rows in a
    wavefront's registers (up to 2560 candidates) and long rows with the
    workgroup radix select. D = 64, one head, random bf16 Q/K; every row
    against the oracle, and (static) bit-exact against the oracle's selection
    on the kernel's own scores."""
    import torch
    G.log(f"[select] long rows {mode}")
    rng = np.random.default_rng(2560)
    S, D, Bs = 96000, 64, 32
    bits = workloads.bf16_bits(rng.standard_normal((2, 1, 1, S, D)).astype(np.float32))
    q, k = (torch.from_numpy(np.ascontiguousarray(bits[i])).view(torch.bfloat16).cuda() for i in range(2))
    f64 = (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    cand = G.dr().build_candidates(G.dr().radial_cfg(4, 24000, Bs, 1.0, 4.0))
    rp, cols = G.host_csr(cand)
    n = np.diff(rp)
    assert (n <= 2560).any() and (n > 2560).any(), (n.min(), n.max())
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau, return_scores=True)
    gs = kept.scores.cpu().numpy()
    s = O.block_scores(O.pool_blocks(f64[0, 0, 0], Bs), O.pool_blocks(f64[1, 0, 0], Bs), rp, cols)
    np.testing.assert_allclose(gs, s, rtol=1e-5, atol=G.SCORE_ATOL)
    ora, margins = O.select_all(s, rp, cols, mode, ratio=ratio, tau=tau)
    gl = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, 0)
    dec, nondec = G.check_selection(gl, ora, margins, s, rp, cols, mode, ratio, tau)
    G.log(f"   rows of {n.min()}..{n.max()} candidates ({(n > 2560).sum()} above 2560): decisive {dec}, "
          f"within-margin {nondec}")
    if mode == "static":
        _static_exact_on_gpu_scores(gl, gs, rp, cols, ratio)
