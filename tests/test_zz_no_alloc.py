"""dr_query_groups_noalloc (the grouping choice on the library's per-GPU
scratch array, for callers that cannot allocate) against dr_query_groups
(caller workspace), through the C ABI: identical modes on two calls in a row,
the second on a smaller input (40 heads, then 12), and both equal to the
choice recomputed on the host from the kept lists."""
import ctypes

import numpy as np
import pytest

import workloads
from tests import gpu_common as G
from tests.test_gpu_groups import _expected_modes, _host_union_totals

pytestmark = pytest.mark.gpu


def _both(name, mode, ratio, tau):
    import torch
    from block_sparse_attention_candidates_amd import _lib as L
    w = workloads.get_workload(name)
    q, k, _ = G.device_qkv(name)
    cand = G.candidates(name)
    kept = G.dr().score_select(q, k, cand, mode=mode, ratio=ratio, tau=tau)
    dims = L.Dims(w.batch, w.heads, w.head_dim, 0)
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    lib = L.lib()
    need = ctypes.c_size_t(0)
    L.check(lib.dr_query_groups_workspace(ctypes.byref(dims), ctypes.byref(need)))
    ws = torch.empty(need.value, dtype=torch.uint8, device="cuda")
    ref = torch.full((w.batch * w.heads,), -7, dtype=torch.int32, device="cuda")
    got = torch.full_like(ref, -7)
    L.check(lib.dr_query_groups(ctypes.byref(dims), ctypes.byref(cand.cfg), cand.row_ptr.data_ptr(), cand.nnz,
                                kept.kept_col.data_ptr(), kept.kept_cnt.data_ptr(), ref.data_ptr(), ws.data_ptr(),
                                ws.numel(), stream))
    L.check(lib.dr_query_groups_noalloc(ctypes.byref(dims), ctypes.byref(cand.cfg), cand.row_ptr.data_ptr(),
                                        cand.nnz, kept.kept_col.data_ptr(), kept.kept_cnt.data_ptr(), got.data_ptr(),
                                        stream))
    torch.cuda.synchronize()
    return w, cand, kept, ref.cpu().numpy(), got.cpu().numpy()


def test_noalloc_grouping_matches_workspace_form_on_two_calls():
    G.log("[no-alloc] grouping choice: wan14b_720p static (40 heads), then wan13b_480p dynamic (12 heads)")
    for name, mode, ratio, tau in (("wan14b_720p", "static", 0.15, 1.0), ("wan13b_480p", "dynamic", 1.0, 0.8)):
        w, cand, kept, ref, got = _both(name, mode, ratio, tau)
        np.testing.assert_array_equal(got, ref, err_msg=f"{name} {mode}")
        assert (got >= 0).all() and (got < 3).all()
        if w.heads <= 12:
            tot, counts = _host_union_totals(kept, cand, w.batch, w.heads)
            np.testing.assert_array_equal(got, _expected_modes(tot, counts), err_msg=f"{name} {mode}: host choice")
        G.log(f"   {name} {mode}: modes {np.bincount(got, minlength=3).tolist()}")
