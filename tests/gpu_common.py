"""Shared helpers of the GPU parity tests: device inputs, oracle references,
the acceptance checks (margin rule, rel-L2 / max-abs), cached per session."""
import hashlib
import json
import math
import os
import sys

import numpy as np

import workloads
from oracle import dynrad_oracle as O

HERE = os.path.dirname(os.path.abspath(__file__))
GOLDEN = os.path.join(HERE, "golden", "candidates.json")

MARGIN = 1e-5           # decisive rows: oracle margin at the cut above this
REL_L2 = 1e-2           # attention output tolerances for bf16 inputs
MAX_ABS = 2e-2
SCORE_ATOL = 2e-5       # float32 block scores vs float64 oracle

_cache = {}


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def golden():
    with open(GOLDEN) as f:
        return json.load(f)["workloads"]


def digest(a):
    return hashlib.sha256(np.ascontiguousarray(a, dtype="<i4").tobytes()).hexdigest()


def dr():
    import block_sparse_attention_candidates_amd as m
    return m


def cfg_of(w):
    return dr().radial_cfg(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam, w.theta_c, w.theta_m)


def host_qkv(name):
    """uint16 bf16 patterns of every head, cached."""
    key = ("host", name)
    if key not in _cache:
        w = workloads.get_workload(name)
        _cache[key] = workloads.qkv_bits_parallel(w, workers=16)
    return _cache[key]


def device_qkv(name):
    import torch
    key = ("dev", name)
    if key not in _cache:
        _cache[key] = tuple(torch.from_numpy(x).view(torch.bfloat16).cuda() for x in host_qkv(name))
    return _cache[key]


def head_f64(name, b, h):
    """Oracle inputs of one head: the same bf16 values as float64 [S, D]."""
    out = []
    for x in host_qkv(name):
        out.append((x[b, h].astype(np.uint32) << 16).view(np.float32).astype(np.float64))
    return out


def candidates(name):
    key = ("cand", name)
    if key not in _cache:
        _cache[key] = dr().build_candidates(cfg_of(workloads.get_workload(name)))
    return _cache[key]


def host_csr(cand):
    return cand.row_ptr.cpu().numpy().astype(np.int64), cand.cols.cpu().numpy().astype(np.int64)


def kept_lists(kept, row_ptr, nnz, Sb, bh):
    col = kept.kept_col.cpu().numpy()
    cnt = kept.kept_cnt.cpu().numpy()
    base = bh * nnz
    return [col[base + row_ptr[a]: base + row_ptr[a] + cnt[bh * Sb + a]].astype(np.int64) for a in range(Sb)]


def oracle_head_selection(name, b, h, mode, ratio, tau, row_ptr, cols):
    """Oracle scores, kept lists and margins of one head (cached)."""
    key = ("sel", name, b, h, mode, ratio, tau)
    if key not in _cache:
        w = workloads.get_workload(name)
        q, k, _ = head_f64(name, b, h)
        s = O.block_scores(O.pool_blocks(q, w.block_size), O.pool_blocks(k, w.block_size), row_ptr, cols)
        kept, margins = O.select_all(s, row_ptr, cols, mode, ratio=ratio, tau=tau)
        _cache[key] = (s, kept, margins)
    return _cache[key]


def check_selection(gpu_lists, ora_lists, margins, scores, row_ptr, cols, mode, ratio, tau):
    """Bit-exact kept lists on decisive rows; on the others the GPU list must be
    a valid selection under the oracle's scores (count / mass within 1e-5).
    Returns (decisive rows, non-decisive rows)."""
    dec = nondec = 0
    for a, (g, o) in enumerate(zip(gpu_lists, ora_lists)):
        assert np.all(np.diff(g) > 0), f"row {a}: kept list not strictly ascending"
        lo, hi = row_ptr[a], row_ptr[a + 1]
        rc, rs = cols[lo:hi], scores[lo:hi]
        assert np.isin(g, rc).all(), f"row {a}: kept block outside the candidate set"
        if margins[a] > MARGIN:
            dec += 1
            assert np.array_equal(g, o), f"row {a} (margin {margins[a]:.3g}): gpu {g[:8]}.. != oracle {o[:8]}.."
        else:
            nondec += 1
            n = len(rc)
            if mode == "static":
                assert len(g) == O.static_count(n, ratio), f"row {a}: count"
                m = np.isin(rc, g)
                if (~m).any():
                    assert rs[m].min() >= rs[~m].max() - MARGIN
            else:
                p = np.exp(rs - rs.max())
                p /= p.sum()
                m = np.isin(rc, g)
                mass = p[m].sum()
                assert mass >= tau - MARGIN, f"row {a}: mass {mass} < tau"
                if len(g) > 1:
                    assert mass - p[m].min() < tau + MARGIN
    return dec, nondec


def rel_l2(x, ref):
    return float(np.linalg.norm(x - ref) / max(np.linalg.norm(ref), 1e-30))


def check_close(x, ref, what=""):
    r = rel_l2(x, ref)
    m = float(np.abs(x - ref).max()) if x.size else 0.0
    assert r <= REL_L2 and m <= MAX_ABS, f"{what}: rel-L2 {r:.3g} max-abs {m:.3g}"
    return r, m


def to_np(t):
    import torch
    return t.float().cpu().numpy() if t.dtype == torch.bfloat16 else t.cpu().numpy()


def sample_blocks(Sb, n, seed):
    rng = np.random.default_rng(seed)
    picks = set(rng.choice(Sb, size=min(n, Sb), replace=False).tolist())
    picks |= {0, Sb - 1}
    return sorted(picks)


def sampled_heads(w):
    hs = {0, w.heads // 2, w.heads - 1} | set(w.periodic_heads())
    return sorted(hs)
