"""Query-block grouping of the sparse attention on the GPU.

The grouping changes which workgroup computes a query block and so the order
in which its kept blocks are accumulated (a workgroup streams its union in an
order that depends on all of its query blocks). dr_sparse_attn_grouped must
therefore agree with dr_sparse_attn within the attention tolerances (and with
the oracle on sampled rows), for every grouping mode, mixed modes per (b, h)
and out-of-range mode values, and be bitwise reproducible for a given
grouping. dr_query_groups must pick, per (b, h), the mode whose groups'
kept-list unions have the smallest estimated total size (groups 0, 4, 8, ...
measured, the sum scaled to the mode's group count; ties to the lower mode),
recomputed here on the host from the kept lists and the host group tables."""
import numpy as np
import pytest

import workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _random_kept(B, H, Sb, cand, rng, empty_frac=0.1):
    rp, cols = G.host_csr(cand)
    lists = {}
    for b in range(B):
        for h in range(H):
            rows = []
            for a in range(Sb):
                c = cols[rp[a]:rp[a + 1]]
                if rng.random() < empty_frac:
                    rows.append(np.zeros(0, dtype=np.int64))
                    continue
                keep = rng.random(len(c)) < rng.uniform(0.05, 0.6)
                rows.append(np.sort(c[keep]).astype(np.int64))
            lists[(b, h)] = rows
    return G.dr().kept_from_lists(lists, rp, B, H)


def _host_union_totals(kept, cand, B, H):
    rp, _ = G.host_csr(cand)
    Sb = cand.num_blocks
    tables = [G.dr().group_table(cand, m) for m in range(3)]
    tot = np.zeros((B * H, 3), dtype=np.int64)
    for bh in range(B * H):
        lists = G.kept_lists(kept, rp, cand.nnz, Sb, bh)
        for m, t in enumerate(tables):
            for g in t[::4]:
                bl = [lists[a] for a in g if a >= 0]
                if bl:
                    tot[bh, m] += len(np.unique(np.concatenate(bl)))
    return tot, [len(t) for t in tables]


def _expected_modes(tot, counts):
    """Smallest tot_m * count_m / sampled_m, by exact rational comparison."""
    from fractions import Fraction
    out = []
    for row in tot:
        est = [Fraction(int(row[m]) * c, -(-c // 4)) if c else None for m, c in enumerate(counts)]
        best = 0
        for m in (1, 2):
            if est[m] is not None and est[m] < est[best]:
                best = m
        out.append(best)
    return np.array(out)


def _same_within_tolerance(out, ref, what):
    """Two GPU outputs that each meet the oracle bar (rel-L2 1e-2, max-abs
    2e-2) differ by at most twice the max-abs bar: bf16 outputs of magnitude 4
    to 8 round to steps of 2^-5, so one rounding step apart is 0.031."""
    a, b = G.to_np(out).ravel(), G.to_np(ref).ravel()
    assert np.isfinite(a).all(), f"{what}: non-finite output"
    r, m = G.rel_l2(a, b), float(np.abs(a - b).max())
    assert r <= G.REL_L2 and m <= 2 * G.MAX_ABS, f"{what}: rel-L2 {r:.3g} max-abs {m:.3g}"


def _check(q, k, v, cand, kept, B, H, label):
    import torch
    ref = G.dr().sparse_attn(q, k, v, cand, kept)
    assert torch.equal(G.dr().sparse_attn(q, k, v, cand, kept), ref), f"{label}: not reproducible"
    variants = {f"mode {m}": torch.full((B * H,), m, dtype=torch.int32, device="cuda") for m in range(3)}
    variants["mixed"] = (torch.arange(B * H, dtype=torch.int32, device="cuda") % 3).to(torch.int32)
    variants["out of range"] = torch.tensor([7, -1, 3] * (B * H), dtype=torch.int32, device="cuda")[:B * H]
    for name, modes in variants.items():
        out = G.dr().sparse_attn(q, k, v, cand, kept, groups=modes)
        _same_within_tolerance(out, ref, f"{label}: {name} vs the consecutive grouping")
        assert torch.equal(G.dr().sparse_attn(q, k, v, cand, kept, groups=modes), out), f"{label}: {name} not reproducible"
    chosen = G.dr().query_groups(q, cand, kept)
    out = G.dr().sparse_attn(q, k, v, cand, kept, groups=chosen)
    _same_within_tolerance(out, ref, f"{label}: chosen grouping")
    tot, counts = _host_union_totals(kept, cand, B, H)
    exp = _expected_modes(tot, counts)
    got = chosen.cpu().numpy()
    np.testing.assert_array_equal(got, exp, err_msg=f"{label}: chosen modes")
    G.log(f"   {label}: modes {np.bincount(got, minlength=3).tolist()}, union totals of head 0 {tot[0].tolist()}")


@pytest.mark.parametrize("name,mode,ratio,tau", [("wan13b_480p", "static", 0.2, 1.0),
                                                 ("wan13b_480p", "dynamic", 1.0, 0.8),
                                                 ("hunyuan_720p", "static", 0.1, 1.0)])
def test_grouping_workload_masks(name, mode, ratio, tau):
    G.log(f"[groups] {name} {mode}")
    w = workloads.get_workload(name)
    q, k, v = G.device_qkv(name)
    cand = G.candidates(name)
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau)
    _check(q, k, v, cand, kept, w.batch, w.heads, f"{name}/{mode}")


@pytest.mark.parametrize("B,H,Nf,Nt,D,Bs", [(2, 3, 6, 200, 128, 64), (1, 2, 10, 300, 128, 128),
                                             (2, 2, 9, 250, 64, 32), (1, 3, 13, 31, 64, 32)])
def test_grouping_random_masks(B, H, Nf, Nt, D, Bs):
    """Random kept lists (about 10% empty rows) on layouts where blocks straddle
    frames, incl. B_s > N_t (13 frames of 31 tokens)."""
    import torch
    G.log(f"[groups] random B={B} H={H} Nf={Nf} Nt={Nt} D={D} Bs={Bs}")
    rng = np.random.default_rng(Nf * 1000 + Nt)
    S = Nf * Nt
    bits = workloads.bf16_bits(rng.standard_normal((3, B, H, S, D)).astype(np.float32))
    q, k, v = (torch.from_numpy(np.ascontiguousarray(bits[i])).view(torch.bfloat16).cuda() for i in range(3))
    cand = G.dr().build_candidates(G.dr().radial_cfg(Nf, Nt, Bs, 1.5, 1.0))
    kept = _random_kept(B, H, cand.num_blocks, cand, rng)
    _check(q, k, v, cand, kept, B, H, f"random {Nf}x{Nt}/{Bs}")


def test_grouping_choice_full_size_static():
    """wan14b_720p with the static 15% selection: the choice on every head
    (host union totals on three heads), and the grouped output within the
    attention tolerances of the consecutive one and of the oracle."""
    import torch
    G.log("[groups] wan14b_720p static")
    name = "wan14b_720p"
    w = workloads.get_workload(name)
    q, k, v = G.device_qkv(name)
    cand = G.candidates(name)
    kept = G.dr().score_select(q, k, cand, mode="static", ratio=0.15)
    chosen = G.dr().query_groups(q, cand, kept)
    ref = G.dr().sparse_attn(q, k, v, cand, kept)
    out = G.dr().sparse_attn(q, k, v, cand, kept, groups=chosen)
    _same_within_tolerance(out, ref, "wan14b_720p static: chosen grouping")
    rp, _ = G.host_csr(cand)
    # sampled rows of the grouped output against the oracle on the GPU's own mask
    from oracle import dynrad_oracle as O
    o = G.to_np(out[0])
    for h in (0, w.heads - 1):
        qh, kh, vh = G.head_f64(name, 0, h)
        blocks = G.sample_blocks(cand.num_blocks, 12, seed=77 + h)
        rows = np.concatenate([np.arange(a * w.block_size, min((a + 1) * w.block_size, w.seq_len)) for a in blocks])
        ref_o = O.sparse_attention_rows(qh, kh, vh, w.block_size, G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h),
                                        blocks)
        G.check_close(o[h][rows], ref_o, f"grouped head {h} vs oracle")
    tables = [G.dr().group_table(cand, m) for m in range(3)]
    got = chosen.cpu().numpy()
    for h in (0, w.heads // 2, w.heads - 1):
        lists = G.kept_lists(kept, rp, cand.nnz, cand.num_blocks, h)
        tot = np.array([[sum(len(np.unique(np.concatenate([lists[a] for a in g if a >= 0])))
                             for g in t[::4] if (g >= 0).any()) for t in tables]])
        best = int(_expected_modes(tot, [len(t) for t in tables])[0])
        assert got[h] == best, (h, tot, got[h])
        full = [sum(len(np.unique(np.concatenate([lists[a] for a in g if a >= 0]))) for g in t if (g >= 0).any())
                for t in tables]
        G.log(f"   head {h}: sampled union totals {tot[0].tolist()}, full {full} -> mode {got[h]}")


@pytest.mark.parametrize("name,mode,ratio,tau", [("wan14b_720p", "static", 0.15, 1.0),
                                                 ("wan14b_720p", "dynamic", 1.0, 0.8)])
def test_every_output_row_written(name, mode, ratio, tau):
    """Output pre-filled with NaN: at the benchmark's launch sizes every row of
    every head is written (by the workgroup that owns its query block) under
    each grouping mode and the kernel's remapping of workgroups to XCDs; the
    dense kernel likewise."""
    import torch
    G.log(f"[groups] every row written: {name} {mode}")
    w = workloads.get_workload(name)
    q, k, v = G.device_qkv(name)
    cand = G.candidates(name)
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau)
    for m in (None, 0, 1, 2):
        groups = None if m is None else torch.full((w.batch * w.heads,), m, dtype=torch.int32, device="cuda")
        out = torch.full_like(q, float("nan"))
        G.dr().sparse_attn(q, k, v, cand, kept, out=out, groups=groups)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), f"rows left unwritten with grouping {m}"
    if mode == "static":
        out = torch.full_like(q, float("nan"))
        G.dr().attn(q, k, v, out=out)
        torch.cuda.synchronize()
        assert not torch.isnan(out).any().item(), "dense: rows left unwritten"
