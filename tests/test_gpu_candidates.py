"""GPU parity of dr_build_candidates against the oracle: bit-exact CSR."""
import numpy as np
import pytest

import workloads
from oracle import dynrad_oracle as O
from tests import gpu_common as G
from tests.test_oracle_candidates import CASES

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name", list(workloads.WORKLOADS))
def test_candidates_full_size_match_golden(name):
    G.log(f"[candidates] {name}")
    gold = G.golden()[name]
    cand = G.candidates(name)
    rp, cols = G.host_csr(cand)
    assert cand.nnz == gold["nnz"] and cand.num_blocks == gold["num_blocks"]
    assert G.digest(rp) == gold["row_ptr_sha256"]
    assert G.digest(cols) == gold["cols_sha256"]


# the oracle's small cases at the block sizes the library builds (32, 64, 128)
@pytest.mark.parametrize("case", [c for c in CASES if c[2] in (32, 64, 128)] + [(3, 256, 32, 1.0, 0.1, 0.0, 0.0), (1, 100, 64, 1.0, 1.0, 0.0, 0.0),
                                          (40, 33, 32, 1.5, 0.05, 0.0, 0.0), (12, 500, 64, 0.9, 0.3, 0.3, 0.4),
                                          (10, 100, 128, 1.0, 0.3, 0.0, 0.0), (6, 200, 128, 1.4, 0.7, 0.45, 0.7)])
def test_candidates_small_exact(case):
    G.log(f"[candidates] small {case}")
    cand = G.dr().build_candidates(G.dr().radial_cfg(*case))
    rp, cols = G.host_csr(cand)
    orp, ocols = O.candidate_csr(*case)
    np.testing.assert_array_equal(rp, orp)
    np.testing.assert_array_equal(cols, ocols)


def test_candidates_capacity_and_async():
    import ctypes
    import torch
    from block_sparse_attention_candidates_amd import _lib as L
    G.log("[candidates] capacity")
    cfg = G.dr().radial_cfg(21, 1560, 32, 1.0, 4.0)
    Sb = G.dr().num_blocks(cfg)
    rp = torch.zeros(Sb + 1, dtype=torch.int32, device="cuda")
    cols = torch.full((1000,), -7, dtype=torch.int32, device="cuda")
    nnz = ctypes.c_int64(0)
    st = L.lib().dr_build_candidates(ctypes.byref(cfg), rp.data_ptr(), cols.data_ptr(), 1000, ctypes.byref(nnz), None)
    assert st == L.DR_ERR_CAPACITY and nnz.value == 424938
    # the first cap entries are the true prefix
    first = G.host_csr(G.candidates("wan13b_480p"))[1][:1000]
    np.testing.assert_array_equal(cols.cpu().numpy(), first)
    # asynchronous form: no count returned, row_ptr[S_b] holds it
    cols = torch.empty(424938, dtype=torch.int32, device="cuda")
    st = L.lib().dr_build_candidates(ctypes.byref(cfg), rp.data_ptr(), cols.data_ptr(), 424938, None, None)
    assert st == L.DR_OK
    torch.cuda.synchronize()
    assert int(rp[-1].item()) == 424938
