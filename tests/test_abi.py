"""CPU checks of the C-ABI library (include/dynrad.h): it loads, exports every
declared entry point, its host per-distance table equals the oracle's, and
invalid calls are rejected by argument validation before any HIP call (no GPU
is touched by these tests)."""
import ctypes
import os
import re

import numpy as np
import pytest

from oracle import dynrad_oracle as O
import workloads

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "dynrad.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dr_[a-z_]+)\s*\(", text)))


def test_exports_every_declared_symbol(dynrad_lib):
    names = declared_functions()
    assert {"dr_build_candidates", "dr_score_select", "dr_sparse_attn", "dr_attn"} <= set(names)
    for n in names:
        assert hasattr(dynrad_lib, n), n


def _cfg(Nf, Nt, Bs, gamma, lam, tc=0.0, tm=0.0):
    import block_sparse_attention_candidates_amd as dr
    return dr.radial_cfg(Nf, Nt, Bs, gamma, lam, tc, tm)


def test_host_table_equals_oracle(dynrad_lib):
    import block_sparse_attention_candidates_amd as dr
    rng = np.random.default_rng(0)
    cases = [(21, 1560, 32, 0.7, 2.0), (21, 3600, 32, 1.0, 4.0), (33, 3600, 64, 1.0, 4.0), (4, 64, 32, 1.0, 2.0),
             (20, 256, 32, 1.0, 0.25), (3, 128, 32, 1.265625, 1.0), (3, 256, 32, 1.0, 0.1)]
    for _ in range(300):
        cases.append((int(rng.integers(1, 100)), int(rng.integers(1, 5000)), int(rng.choice([32, 64])),
                      float(rng.uniform(0.05, 4.0)), float(rng.choice([0.0, rng.uniform(0.0, 2.0)]))))
    # round-number parameters hit exact ties of Eqs. 3 and 5
    for g in (0.5, 0.75, 1.0, 1.25, 1.5, 2.0, 3.0):
        for lam in (0.0625, 0.125, 0.25, 0.5, 1.0):
            cases.append((64, 1000, 32, g, lam))
    for Nf, Nt, Bs, g, lam in cases:
        if Nf * Nt > 16384 * Bs:
            continue
        w, sf = dr.distance_table(_cfg(Nf, Nt, Bs, g, lam))
        wo, sfo = O.distance_table(Nf, Nt, Bs, g, lam)
        np.testing.assert_array_equal(np.minimum(w, 1 << 30), np.minimum(wo, 1 << 30), err_msg=str((Nf, Nt, Bs, g, lam)))
        np.testing.assert_array_equal(sf, np.minimum(sfo, 1 << 30), err_msg=str((Nf, Nt, Bs, g, lam)))


def test_num_blocks(dynrad_lib):
    import block_sparse_attention_candidates_amd as dr
    for name, w in workloads.WORKLOADS.items():
        assert dr.num_blocks(_cfg(w.num_frames, w.tokens_per_frame, w.block_size, w.gamma, w.lam)) == w.num_blocks


FAKE = ctypes.c_void_p(4096)     # never dereferenced: validation fails first


def test_radial_validation(dynrad_lib):
    from block_sparse_attention_candidates_amd import _lib as L
    bad = [(_cfg(4, 64, 256, 1.0, 2.0), L.DR_ERR_UNSUPPORTED),      # B_s = 256 not built
           (_cfg(4, 64, 48, 1.0, 2.0), L.DR_ERR_UNSUPPORTED),       # B_s must be 32, 64 or 128
           (_cfg(4, 64, 0, 1.0, 2.0), L.DR_ERR_INVALID_ARG),
           (_cfg(0, 64, 32, 1.0, 2.0), L.DR_ERR_INVALID_ARG),
           (_cfg(4, 64, 32, 0.0, 2.0), L.DR_ERR_INVALID_ARG),         # gamma must be > 0
           (_cfg(4, 64, 32, 1.0, -1.0), L.DR_ERR_INVALID_ARG),
           (_cfg(4, 64, 32, 1.0, 2.0, 1.5, 0.0), L.DR_ERR_INVALID_ARG),
           (_cfg(4, 64, 32, 1.0, 2.0, 0.0, -0.1), L.DR_ERR_INVALID_ARG),
           (_cfg(4, 64, 32, float("nan"), 2.0), L.DR_ERR_INVALID_ARG),
           (_cfg(5000, 64, 32, 1.0, 2.0), L.DR_ERR_UNSUPPORTED),      # N_f above 4096
           (_cfg(100, 10000, 32, 1.0, 2.0), L.DR_ERR_UNSUPPORTED)]    # S_b above 16384
    for cfg, want in bad:
        assert dynrad_lib.dr_num_blocks(ctypes.byref(cfg)) == -want
        nnz = ctypes.c_int64(-1)
        assert dynrad_lib.dr_build_candidates(ctypes.byref(cfg), FAKE, FAKE, 10, ctypes.byref(nnz), None) == want
        assert dynrad_lib.dr_last_error().decode() != ""
    assert dynrad_lib.dr_num_blocks(ctypes.byref(_cfg(4, 64, 128, 1.0, 2.0))) == 2   # B_s = 128 is built
    cfg = _cfg(4, 64, 32, 1.0, 2.0)
    cfg.reserved = 1
    assert dynrad_lib.dr_num_blocks(ctypes.byref(cfg)) == -L.DR_ERR_INVALID_ARG
    good = _cfg(4, 64, 32, 1.0, 2.0)
    assert dynrad_lib.dr_build_candidates(ctypes.byref(good), None, FAKE, 10, None, None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_build_candidates(ctypes.byref(good), FAKE, FAKE, 0, None, None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_build_candidates(None, FAKE, FAKE, 10, None, None) == L.DR_ERR_INVALID_ARG


def test_select_and_attention_validation(dynrad_lib):
    from block_sparse_attention_candidates_amd import _lib as L
    cfg = _cfg(4, 64, 32, 1.0, 2.0)            # S = 256, S_b = 8
    dims = L.Dims(1, 2, 64, 0)
    sel = L.SelectCfg(L.DR_STATIC_RATIO, 0, 0.5, 0.8)
    size = ctypes.c_size_t(0)
    assert dynrad_lib.dr_score_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(sel), 64,
                                                ctypes.byref(size)) == L.DR_OK
    # pooled Q and K: 2 * (1*2*8*64*4 = 4096 B) + scores 1*2*64*4 = 512 B + the tile map of one group of
    # 32 query blocks (count, tile words, bitmaps, positions: 4 parts), each rounded up to 256 B
    assert size.value == 4096 + 4096 + 512 + 4 * 256
    fused = L.SelectCfg(L.DR_DYNAMIC_THRESHOLD, 1, 0.5, 0.8)
    assert dynrad_lib.dr_score_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(fused), 64,
                                                ctypes.byref(size)) == L.DR_OK
    assert size.value == 2048 + 2048 + 256 + 4 * 256

    def ss(d=dims, s=sel, nnz=64, ws_bytes=1 << 20, q=FAKE):
        return dynrad_lib.dr_score_select(ctypes.byref(d), ctypes.byref(cfg), ctypes.byref(s), q, FAKE, FAKE, FAKE,
                                          nnz, FAKE, FAKE, None, FAKE, ws_bytes, None)
    assert ss(s=L.SelectCfg(L.DR_STATIC_RATIO, 0, 0.0, 0.8)) == L.DR_ERR_INVALID_ARG     # ratio 0
    assert ss(s=L.SelectCfg(L.DR_STATIC_RATIO, 0, 1.5, 0.8)) == L.DR_ERR_INVALID_ARG     # ratio > 1
    assert ss(s=L.SelectCfg(L.DR_DYNAMIC_THRESHOLD, 0, 0.5, 0.0)) == L.DR_ERR_INVALID_ARG  # tau 0
    assert ss(s=L.SelectCfg(L.DR_DYNAMIC_THRESHOLD, 0, 0.5, 1.5)) == L.DR_ERR_INVALID_ARG
    assert ss(s=L.SelectCfg(7, 0, 0.5, 0.8)) == L.DR_ERR_INVALID_ARG
    assert ss(s=L.SelectCfg(L.DR_STATIC_RATIO, 3, 0.5, 0.8)) == L.DR_ERR_INVALID_ARG     # score_heads > H
    assert ss(d=L.Dims(1, 2, 96, 0)) == L.DR_ERR_UNSUPPORTED
    assert ss(d=L.Dims(0, 2, 64, 0)) == L.DR_ERR_INVALID_ARG
    assert ss(nnz=0) == L.DR_ERR_INVALID_ARG
    assert ss(nnz=65) == L.DR_ERR_INVALID_ARG                                           # > S_b^2
    assert ss(q=None) == L.DR_ERR_INVALID_ARG
    assert ss(ws_bytes=100) == L.DR_ERR_CAPACITY

    def sa(d=dims, nnz=64, out=ctypes.c_void_p(8192), scale=0.125):
        return dynrad_lib.dr_sparse_attn(ctypes.byref(d), ctypes.byref(cfg), FAKE, ctypes.c_void_p(4096 + 64),
                                         ctypes.c_void_p(4096 + 128), FAKE, nnz, FAKE, FAKE, scale, out, None)
    assert sa(out=FAKE) == L.DR_ERR_INVALID_ARG            # aliases q
    assert sa(out=None) == L.DR_ERR_INVALID_ARG
    assert sa(d=L.Dims(1, 2, 32, 0)) == L.DR_ERR_UNSUPPORTED
    assert sa(nnz=0) == L.DR_ERR_INVALID_ARG
    assert sa(scale=float("inf")) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_attn(ctypes.byref(dims), 0, FAKE, FAKE, FAKE, ctypes.c_float(0.1), ctypes.c_void_p(8192),
                              None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_attn(ctypes.byref(L.Dims(1, 1, 80, 0)), 10, FAKE, FAKE, FAKE, ctypes.c_float(0.1),
                              ctypes.c_void_p(8192), None) == L.DR_ERR_UNSUPPORTED
    for s in range(5):
        assert dynrad_lib.dr_status_string(s).decode()


def test_token_select_validation(dynrad_lib):
    """dr_token_select rejects out-of-range configurations before any HIP call,
    and its workspace is the sum of its aligned parts."""
    from block_sparse_attention_candidates_amd import _lib as L
    FAKE = ctypes.c_void_p(4096)
    cfg = _cfg(4, 64, 32, 1.0, 2.0)             # S = 256, S_b = 8
    dims = L.Dims(1, 2, 64, 0)
    tok = L.TokenCfg(2, 0, -1.5, 2.0, 1e-6)
    size = ctypes.c_size_t(0)
    assert dynrad_lib.dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(tok), 64,
                                                ctypes.byref(size)) == L.DR_OK
    # partials: 1 workgroup x 4 key-range splits x FR (255 // 64 + 2 = 5) x N_f 4 x 32 B = 2560;
    # thr 64 B -> 256; maxima 128 B -> 256; counts 128 B -> 256; served 64 B -> 256; flags 64 B -> 256;
    # B_s = 32: column sums 64 entries x 32 columns x 8 B = 16384; undecided marks 64 B -> 256
    assert size.value == 2560 + 5 * 256 + 16384 + 256
    cfg64 = _cfg(4, 64, 64, 1.0, 2.0)           # B_s = 64: four 32 x 32 tiles' column sums per entry
    assert dynrad_lib.dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cfg64), ctypes.byref(tok), 16,
                                                ctypes.byref(size)) == L.DR_OK
    assert size.value == 2560 + 5 * 256 + 16 * 4 * 32 * 8 + 256
    cfg128 = _cfg(4, 64, 128, 1.0, 2.0)         # B_s = 128: the ring mark pass, no column sums
    assert dynrad_lib.dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cfg128), ctypes.byref(tok), 4,
                                                ctypes.byref(size)) == L.DR_OK
    assert size.value == 2560 + 5 * 256

    def ts(d=dims, c=cfg, t=tok, nnz=64, ws_bytes=1 << 20, q=FAKE):
        return dynrad_lib.dr_token_select(ctypes.byref(d), ctypes.byref(c), ctypes.byref(t), q, FAKE, FAKE, FAKE,
                                          nnz, FAKE, FAKE, FAKE, ws_bytes, None)
    assert ts(t=L.TokenCfg(3, 0, -1.5, 2.0, 1e-6), d=L.Dims(1, 4, 64, 0)) == L.DR_ERR_UNSUPPORTED  # H_f = 3
    assert ts(t=L.TokenCfg(3, 0, -1.5, 2.0, 1e-6)) == L.DR_ERR_INVALID_ARG    # H_f > heads
    assert ts(t=L.TokenCfg(0, 0, -1.5, 2.0, 1e-6)) == L.DR_ERR_INVALID_ARG
    assert ts(t=L.TokenCfg(2, 1, -1.5, 2.0, 1e-6)) == L.DR_ERR_INVALID_ARG    # reserved
    assert ts(t=L.TokenCfg(2, 0, float("nan"), 2.0, 1e-6)) == L.DR_ERR_INVALID_ARG
    assert ts(t=L.TokenCfg(2, 0, -1.5, 2.0, 0.0)) == L.DR_ERR_INVALID_ARG     # eps must be > 0
    assert ts(c=_cfg(8, 16, 32, 1.0, 2.0)) == L.DR_ERR_UNSUPPORTED            # N_t < 32
    assert ts(c=_cfg(65, 64, 32, 1.0, 2.0)) == L.DR_ERR_UNSUPPORTED           # N_f > 64
    assert ts(q=None) == L.DR_ERR_INVALID_ARG
    assert ts(ws_bytes=100) == L.DR_ERR_CAPACITY
    assert ts(t=L.TokenCfg(2, 0, float("-inf"), float("inf"), 1e-6), ws_bytes=100) == L.DR_ERR_CAPACITY


def test_static_select_validation(dynrad_lib):
    """dr_static_select rejects out-of-range configurations before any HIP call;
    its workspace is 48 + 8192 bytes per ordered frame pair plus the flags."""
    from block_sparse_attention_candidates_amd import _lib as L
    FAKE = ctypes.c_void_p(4096)
    cfg = _cfg(4, 64, 32, 1.0, 2.0)             # S = 256, S_b = 8, 16 frame pairs
    dims = L.Dims(1, 2, 64, 0)
    sc = L.StaticCfg(0.5, 0.3, 7)
    size = ctypes.c_size_t(0)
    assert dynrad_lib.dr_static_select_workspace(ctypes.byref(cfg), 64, ctypes.byref(size)) == L.DR_OK
    # states 16 x 48 = 768; histograms 16 x 8192 = 131072; flags 64 -> 256
    assert size.value == 768 + 131072 + 256

    def ss(d=dims, c=cfg, s=sc, nnz=64, ws_bytes=1 << 20, rp=FAKE):
        return dynrad_lib.dr_static_select(ctypes.byref(d), ctypes.byref(c), ctypes.byref(s) if s else None, rp,
                                           FAKE, nnz, FAKE, FAKE, FAKE, ws_bytes, None)
    assert ss(s=None) == L.DR_ERR_INVALID_ARG
    assert ss(s=L.StaticCfg(1.5, 0.3, 7)) == L.DR_ERR_INVALID_ARG
    assert ss(s=L.StaticCfg(0.5, -0.1, 7)) == L.DR_ERR_INVALID_ARG
    assert ss(s=L.StaticCfg(float("nan"), 0.3, 7)) == L.DR_ERR_INVALID_ARG
    assert ss(c=_cfg(8, 16, 32, 1.0, 2.0)) == L.DR_ERR_UNSUPPORTED            # N_t < 32
    assert ss(c=_cfg(65, 64, 32, 1.0, 2.0)) == L.DR_ERR_UNSUPPORTED           # N_f > 64
    assert ss(nnz=0) == L.DR_ERR_INVALID_ARG
    assert ss(rp=None) == L.DR_ERR_INVALID_ARG
    assert ss(ws_bytes=100) == L.DR_ERR_CAPACITY


def test_proxy_error_validation(dynrad_lib):
    """dr_proxy_error checks pointers, sizes, alignment and workspace before any HIP call."""
    from block_sparse_attention_candidates_amd import _lib as L
    A, B = ctypes.c_void_p(4096), ctypes.c_void_p(8192)

    def pe(r=A, t=B, n=100, cnt=None, n_cnt=0, out=A, ws=B, ws_bytes=L.PROXY_WS_BYTES):
        return dynrad_lib.dr_proxy_error(r, t, n, cnt, n_cnt, out, ws, ws_bytes, None)
    assert pe(r=None) == L.DR_ERR_INVALID_ARG
    assert pe(out=None) == L.DR_ERR_INVALID_ARG
    assert pe(n=0) == L.DR_ERR_INVALID_ARG
    assert pe(n_cnt=5) == L.DR_ERR_INVALID_ARG            # counts without a pointer
    assert pe(t=ctypes.c_void_p(8200)) == L.DR_ERR_INVALID_ARG   # not 16-byte aligned
    assert pe(ws_bytes=L.PROXY_WS_BYTES - 8) == L.DR_ERR_CAPACITY

    def pl(total=100, alpha=10.0, target=0.8, **kw):
        a = dict(r=A, t=B, n=100, cnt=None, n_cnt=0, out=A, ws=B, ws_bytes=L.PROXY_WS_BYTES) | kw
        return dynrad_lib.dr_proxy_loss(a["r"], a["t"], a["n"], a["cnt"], a["n_cnt"], total, alpha, target, a["out"],
                                        a["ws"], a["ws_bytes"], None)
    assert pl(total=0) == L.DR_ERR_INVALID_ARG
    assert pl(alpha=-1.0) == L.DR_ERR_INVALID_ARG
    assert pl(alpha=float("inf")) == L.DR_ERR_INVALID_ARG
    assert pl(target=float("nan")) == L.DR_ERR_INVALID_ARG
    assert pl(r=None) == L.DR_ERR_INVALID_ARG
    assert pl(ws_bytes=16) == L.DR_ERR_CAPACITY


def test_query_groups_noalloc_validation(dynrad_lib):
    """dr_query_groups_noalloc checks its arguments before any HIP call,
    including the (b, h) limit of the library's scratch array."""
    import block_sparse_attention_candidates_amd as dr
    from block_sparse_attention_candidates_amd import _lib as L
    cfg = dr.radial_cfg(4, 64, 32, 1.0, 2.0)
    P = ctypes.c_void_p(4096)

    def call(B=1, H=2, nnz=64, rp=P, kc=P, kn=P, gm=P):
        dims = L.Dims(B, H, 64, 0)
        return dynrad_lib.dr_query_groups_noalloc(ctypes.byref(dims), ctypes.byref(cfg), rp, nnz, kc, kn, gm, None)
    assert call(rp=None) == L.DR_ERR_INVALID_ARG
    assert call(gm=None) == L.DR_ERR_INVALID_ARG
    assert call(nnz=0) == L.DR_ERR_INVALID_ARG
    assert call(B=256, H=256) == L.DR_ERR_UNSUPPORTED          # 65536 (b, h) pairs
    assert b"65535" in dynrad_lib.dr_last_error()


def test_wait_limit_and_report_validation(dynrad_lib):
    """dr_set_wait_limit accepts [0, 2^31); dr_wait_report rejects a NULL
    flags pointer before any HIP call."""
    from block_sparse_attention_candidates_amd import _lib as L
    assert dynrad_lib.dr_set_wait_limit(-1) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_set_wait_limit(1 << 31) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_set_wait_limit(5) == L.DR_OK
    assert dynrad_lib.dr_set_wait_limit(0) == L.DR_OK
    assert dynrad_lib.dr_wait_report(None, None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_status_string(L.DR_ERR_WAIT) == b"bounded wait gave up"


@pytest.mark.parametrize("layout", [(21, 3600, 32), (21, 1560, 32), (33, 3600, 64), (9, 33, 128), (6, 200, 64),
                                    (4, 64, 32), (1, 1000, 32), (13, 31, 32), (5, 300, 128)])
def test_query_group_tables_partition_the_blocks(dynrad_lib, layout):
    """Every grouping mode is a partition of the query blocks into groups of
    256 / B_s slots (-1 = empty), and modes 1 and 2 take F frame rows by R
    adjacent columns, row f being blocks [floor(f N_t / B_s), floor((f + 1) N_t / B_s))
    (the last row up to S_b)."""
    import block_sparse_attention_candidates_amd as dr
    Nf, Nt, Bs = layout
    cand_cfg = _cfg(Nf, Nt, Bs, 1.0, 1.0)
    Sb = dr.num_blocks(cand_cfg)
    Q = 256 // Bs
    shapes = {32: [(4, 2), (2, 4)], 64: [(2, 2), (4, 1)], 128: [(2, 1)]}[Bs]
    starts = [f * Nt // Bs for f in range(Nf)] + [Sb]
    frame_of = np.searchsorted(np.array(starts[1:]), np.arange(Sb), side="right")

    class _C:
        cfg = cand_cfg
    for mode in range(3):
        t = dr.group_table(_C, mode)
        assert t.shape[1] == Q
        if mode == 2 and Bs == 128:
            assert t.size == 0
            continue
        used = t[t >= 0]
        assert np.array_equal(np.sort(used), np.arange(Sb)), f"mode {mode}: not a partition"
        if mode == 0:
            assert np.array_equal(t.reshape(-1)[:Sb], np.arange(Sb))
            continue
        F, R = shapes[mode - 1]
        for g in t:
            chunk = set()
            for s, a in enumerate(g):
                if a < 0:
                    continue
                f = int(frame_of[a])
                c = int(a - starts[f])
                # slot s holds row (chunk row) * F + s // R, column (chunk column) * R + s % R
                assert (f - s // R) % F == 0 and (c - s % R) % R == 0, (mode, g)
                chunk.add(((f - s // R) // F, (c - s % R) // R))
            assert len(chunk) <= 1, (mode, g)
    assert dynrad_lib.dr_query_group_table(ctypes.byref(cand_cfg), 3, None, 0) < 0
    assert dynrad_lib.dr_query_group_table(ctypes.byref(cand_cfg), -1, None, 0) < 0


def test_query_groups_validation(dynrad_lib):
    from block_sparse_attention_candidates_amd import _lib as L
    cfg = _cfg(4, 64, 32, 1.0, 2.0)            # S = 256, S_b = 8
    dims = L.Dims(2, 3, 64, 0)
    size = ctypes.c_size_t(0)
    assert dynrad_lib.dr_query_groups_workspace(ctypes.byref(dims), ctypes.byref(size)) == L.DR_OK
    assert size.value == 256                  # 2 * 3 * 3 * 4 = 72 bytes, rounded up
    args = (ctypes.byref(dims), ctypes.byref(cfg), FAKE, 16, FAKE, FAKE, FAKE)
    assert dynrad_lib.dr_query_groups(*args, FAKE, 255, None) == L.DR_ERR_CAPACITY
    assert dynrad_lib.dr_query_groups(*args, None, 256, None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_query_groups(ctypes.byref(dims), ctypes.byref(cfg), FAKE, 16, FAKE, FAKE, None, FAKE, 256,
                                      None) == L.DR_ERR_INVALID_ARG
    assert dynrad_lib.dr_sparse_attn_grouped(ctypes.byref(dims), ctypes.byref(cfg), FAKE, FAKE, FAKE, FAKE, 16,
                                             FAKE, FAKE, None, 0.125, FAKE, None) == L.DR_ERR_INVALID_ARG
