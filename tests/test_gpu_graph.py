"""The hot path captured in a HIP graph: one step (asynchronous candidate
build, scoring and selection or the token-level selector, the grouping
choice, grouped sparse attention; [DR] §3.1-§3.3) recorded once and replayed
three times, with the program's own eager work (fill kernels overwriting every
output) and synchronisations between the replays. Every replay must equal the
eager step bitwise: the kernels are deterministic and record no memset, copy
or host synchronisation."""
import ctypes
import math

import pytest

import workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _step(name, mode, ratio, tau, taus=None):
    import torch
    from block_sparse_attention_candidates_amd import _lib
    w = workloads.get_workload(name)
    q, k, v = G.device_qkv(name)
    cfg = G.cfg_of(w)
    cand = G.candidates(name)
    L = _lib.lib()
    dims = _lib.Dims(w.batch, w.heads, w.head_dim, 0)
    wsb = ctypes.c_size_t(0)
    if mode == "token":
        tokc = _lib.TokenCfg(2, 0, float(taus[0]), float(taus[1]), 1e-6)
        _lib.check(L.dr_token_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(tokc), cand.nnz,
                                               ctypes.byref(wsb)))
    else:
        selc = G.dr()._select_cfg(mode, ratio, tau, 0)
        _lib.check(L.dr_score_select_workspace(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(selc), cand.nnz,
                                               ctypes.byref(wsb)))
    gwsb = ctypes.c_size_t(0)
    _lib.check(L.dr_query_groups_workspace(ctypes.byref(dims), ctypes.byref(gwsb)))
    dev = dict(device="cuda")
    ws = torch.empty(wsb.value, dtype=torch.uint8, **dev)
    gws = torch.empty(gwsb.value, dtype=torch.uint8, **dev)
    bufs = {
        "row_ptr": torch.empty_like(cand.row_ptr),
        "cols": torch.empty_like(cand.cols),
        "kept_col": torch.empty(w.batch * w.heads * cand.nnz, dtype=torch.int32, **dev),
        "kept_cnt": torch.empty(w.batch * w.heads * cand.num_blocks, dtype=torch.int32, **dev),
        "groups": torch.empty(w.batch * w.heads, dtype=torch.int32, **dev),
        "out": torch.empty_like(q),
    }
    b = bufs
    scale = ctypes.c_float(1.0 / math.sqrt(w.head_dim))

    def stream():
        return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)

    def step():
        _lib.check(L.dr_build_candidates(ctypes.byref(cfg), b["row_ptr"].data_ptr(), b["cols"].data_ptr(), cand.nnz,
                                         None, stream()))
        if mode == "token":
            _lib.check(L.dr_token_select(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(tokc), q.data_ptr(),
                                         k.data_ptr(), b["row_ptr"].data_ptr(), b["cols"].data_ptr(), cand.nnz,
                                         b["kept_col"].data_ptr(), b["kept_cnt"].data_ptr(), ws.data_ptr(),
                                         ws.numel(), stream()))
        else:
            _lib.check(L.dr_score_select(ctypes.byref(dims), ctypes.byref(cfg), ctypes.byref(selc), q.data_ptr(),
                                         k.data_ptr(), b["row_ptr"].data_ptr(), b["cols"].data_ptr(), cand.nnz,
                                         b["kept_col"].data_ptr(), b["kept_cnt"].data_ptr(), None, ws.data_ptr(),
                                         ws.numel(), stream()))
        _lib.check(L.dr_query_groups(ctypes.byref(dims), ctypes.byref(cfg), b["row_ptr"].data_ptr(), cand.nnz,
                                     b["kept_col"].data_ptr(), b["kept_cnt"].data_ptr(), b["groups"].data_ptr(),
                                     gws.data_ptr(), gws.numel(), stream()))
        _lib.check(L.dr_sparse_attn_grouped(ctypes.byref(dims), ctypes.byref(cfg), q.data_ptr(), k.data_ptr(),
                                            v.data_ptr(), b["row_ptr"].data_ptr(), cand.nnz,
                                            b["kept_col"].data_ptr(), b["kept_cnt"].data_ptr(),
                                            b["groups"].data_ptr(), scale, b["out"].data_ptr(), stream()))
    return step, bufs


def _scramble(bufs):
    """Eager work between replays: overwrite every output (fill kernels); the
    kept lists' unused tail gets the same value as before the eager step."""
    import torch
    for key, x in bufs.items():
        if key == "kept_col":
            x.fill_(-1)
        elif x.dtype == torch.bfloat16:
            x.fill_(7.0)
        else:
            x.fill_(-7)


CASES = [("wan13b_480p", "static", 0.2, 1.0, None),
         ("wan13b_480p", "dynamic", 1.0, 0.8, None),
         ("wan13b_480p", "token", 1.0, 1.0, (-1.5, 2.0))]


@pytest.mark.parametrize("name,mode,ratio,tau,taus", CASES)
def test_hot_path_graph_replays_equal_eager(name, mode, ratio, tau, taus):
    import torch
    G.log(f"[graph] {name} {mode}: eager step, capture, 3 replays")
    step, bufs = _step(name, mode, ratio, tau, taus)
    bufs["kept_col"].fill_(-1)
    step()
    torch.cuda.synchronize()
    ref = {key: x.clone() for key, x in bufs.items()}
    assert int(ref["kept_cnt"].sum().item()) > 0
    # warm-up on a side stream (default priority), then capture
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        step()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for r in range(3):
        _scramble(bufs)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for key, x in bufs.items():
            assert torch.equal(x, ref[key]), f"replay {r}: {key} differs from the eager step"
    G.dr().wait_report()
