"""GPU parity of the proxy-task evaluator ([DR] App. C.2 Eq. 20, C.4 Eq. 22):
dr_proxy_error's sums against float64 NumPy, and the penalised loss of whole
masks (dr_attn + dr_sparse_attn on the drift inputs with a random probe, then
dr_proxy_loss) against the oracle's probe form on the same inputs and masks."""
import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits)).view(torch.bfloat16).cuda()


def _f64(bits):
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_proxy_error_sums_exact_and_reproducible():
    """n = 1,000,003 (a ragged tail after the 8-element loads) and 5,001 counts."""
    import torch
    G.log("[proxy] error sums vs float64 NumPy")
    rng = np.random.default_rng(31)
    a = workloads.bf16_bits(rng.standard_normal(1_000_003).astype(np.float32))
    b = workloads.bf16_bits((rng.standard_normal(1_000_003) * 0.5).astype(np.float32))
    cnt = rng.integers(0, 2000, 5001).astype(np.int32)
    kept = G.dr().Kept(torch.zeros(1, dtype=torch.int32, device="cuda"), torch.from_numpy(cnt).cuda())
    r1 = G.dr().proxy_error(_dev(a), _dev(b), kept)
    r2 = G.dr().proxy_error(_dev(a), _dev(b), kept)
    assert r1 == r2
    fa, fb = _f64(a), _f64(b)
    assert r1[0] == pytest.approx(float(((fb - fa) ** 2).sum()), rel=1e-12)
    assert r1[1] == pytest.approx(float((fa ** 2).sum()), rel=1e-12)
    assert r1[2] == float(cnt.sum())
    r3 = G.dr().proxy_error(_dev(a[:7]), _dev(b[:7]))
    assert r3[0] == pytest.approx(float(((fb[:7] - fa[:7]) ** 2).sum()), rel=1e-12) and r3[2] == 0.0


def _oracle_probe(qb, kb, zb, kept_lists_per_head, Bs):
    num = den = 0.0
    for h in range(qb.shape[1]):
        n, d = O.proxy_error_sums(_f64(qb[0, h]), _f64(kb[0, h]), _f64(zb[0, h]), kept_lists_per_head[h], Bs)
        num += n
        den += d
    return num / den


def _check(res, ora_nmse, ora_sparsity, label):
    G.log(f"   {label}: nmse gpu {res['nmse']:.6g} oracle {ora_nmse:.6g}, sparsity {res['sparsity']:.4f}, "
          f"loss {res['loss']:.5g}")
    # bf16 outputs: each element carries ~2^-9 relative rounding, which moves the
    # error sum by a few percent of the signal at these error levels
    assert res["nmse"] == pytest.approx(ora_nmse, rel=0.05, abs=2e-4)
    assert res["sparsity"] == pytest.approx(ora_sparsity, abs=1e-12)
    # the library's Eq. 22 (dr_proxy_loss) on its own terms equals the oracle's formula
    assert res["nmse"] == res["err_sum"] / res["ref_sum"]
    assert res["loss"] == pytest.approx(O.proxy_loss(res["nmse"], res["sparsity"]), rel=1e-12, abs=1e-15)
    # and the loss as a whole is the oracle's loss within the error tolerance above
    assert res["loss"] == pytest.approx(O.proxy_loss(ora_nmse, ora_sparsity), rel=0.05, abs=2e-4)


@pytest.mark.parametrize("regime", ["low", "mid", "high"])
def test_proxy_loss_block_static_mask(regime):
    """Drift inputs of 6 frames of 16x16 tokens, D = 64, 2 heads, B_s = 32,
    block-level static selection (ratio 0.3) on a radial candidate set."""
    G.log(f"[proxy] {regime} drift, block-level static mask")
    delta = workloads.PROXY_DRIFT[regime]
    qb, kb, zb = workloads.proxy_qkz(6, 16, 16, 64, 2, delta, seed=41, as_bits=True)
    q, k, z = _dev(qb), _dev(kb), _dev(zb)
    cand = G.dr().build_candidates(G.dr().radial_cfg(6, 256, 32, 1.0, 2.0))
    kept = G.dr().score_select(q, k, cand, mode="static", ratio=0.3)
    res = G.dr().proxy_loss(q, k, z, cand, kept)
    rp, _ = G.host_csr(cand)
    lists = [G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h) for h in range(2)]
    _check(res, _oracle_probe(qb, kb, zb, lists, 32), O.proxy_sparsity(lists, cand.num_blocks), regime)


def test_proxy_loss_oracle_decay_static_mask():
    """The oracle's decay-state static mask (Table 2 'low' preset), uploaded
    as kept lists: the GPU loss of that exact mask against the oracle's."""
    G.log("[proxy] oracle decay-static mask")
    pr = workloads.STATIC_PRESETS["low"]
    Nf, Nt, Bs = 6, 256, 32
    qb, kb, zb = workloads.proxy_qkz(Nf, 16, 16, 64, 1, 0.15, seed=43, as_bits=True)
    ora_kept = O.static_select(Nf, Nt, Bs, pr["gamma"], pr["lam"], pr["rho_near"], pr["rho_far"], 9,
                               pr["theta_c"], pr["theta_m"])
    cand = G.dr().build_candidates(G.dr().radial_cfg(Nf, Nt, Bs, pr["gamma"], pr["lam"], pr["theta_c"],
                                                     pr["theta_m"]))
    rp, _ = G.host_csr(cand)
    kept = G.dr().kept_from_lists({(0, 0): ora_kept}, rp, 1, 1)
    res = G.dr().proxy_loss(_dev(qb), _dev(kb), _dev(zb), cand, kept)
    _check(res, _oracle_probe(qb, kb, zb, [ora_kept], Bs), O.proxy_sparsity([ora_kept], cand.num_blocks), "low")


def test_proxy_full_mask_is_dense():
    """Every block kept: the sparse kernel reproduces the dense one up to
    rounding, so the normalised error is ~0 and the penalty is the full 8."""
    G.log("[proxy] full mask")
    qb, kb, zb = workloads.proxy_qkz(4, 16, 16, 128, 2, 0.4, seed=47, as_bits=True)
    cand = G.dr().build_candidates(G.dr().radial_cfg(4, 256, 32, 4.0, 2.0))   # window covers every frame
    rp, cols = G.host_csr(cand)
    full = [np.arange(cand.num_blocks)] * cand.num_blocks
    assert all(np.array_equal(cols[rp[a]:rp[a + 1]], full[a]) for a in range(cand.num_blocks))
    kept = G.dr().kept_from_lists({(0, h): full for h in range(2)}, rp, 1, 2)
    res = G.dr().proxy_loss(_dev(qb), _dev(kb), _dev(zb), cand, kept)
    G.log(f"   nmse {res['nmse']:.3g}")
    assert res["sparsity"] == 0.0 and res["nmse"] < 1e-5 and res["loss"] == pytest.approx(8.0, abs=1e-5)
