"""The bounded-wait report (dr_wait_report, dr_set_wait_limit): with the poll
limit lowered from the host to one poll, the ring waits of the attention and
token-selection kernels give up on purpose, every kernel still exits, and the
report names them; with the default limit the same calls report nothing and
give the reference output again."""
import numpy as np
import pytest

import workloads
from tests import gpu_common as G

pytestmark = pytest.mark.gpu


def _limited(fn):
    """fn() under a one-poll limit; returns the flags the report raised with."""
    dr = G.dr()
    from block_sparse_attention_candidates_amd import _lib as L
    assert dr.wait_report() == 0
    dr.set_wait_limit(1)
    try:
        fn()
        with pytest.raises(dr.DynradError) as ei:
            dr.wait_report()
        assert ei.value.status == L.DR_ERR_WAIT
    finally:
        dr.set_wait_limit(0)
    assert dr.wait_report() == 0          # read and cleared
    return int(ei.value.detail.split("flags 0x")[1].split(")")[0], 16)


def test_attention_waits_report_give_ups():
    import torch
    G.log("[wait] attention under a one-poll limit")
    from block_sparse_attention_candidates_amd import _lib as L
    name = "wan13b_480p"
    q, k, v = G.device_qkv(name)
    q, k, v = (x[:, :4].contiguous() for x in (q, k, v))
    cand = G.candidates(name)
    kept = G.dr().score_select(q, k, cand, mode="static", ratio=0.5)
    ref = G.dr().sparse_attn(q, k, v, cand, kept)
    ref_d = G.dr().attn(q[:, :1], k[:, :1], v[:, :1])
    assert G.dr().wait_report() == 0
    flags = _limited(lambda: (G.dr().sparse_attn(q, k, v, cand, kept), G.dr().attn(q[:, :1], k[:, :1], v[:, :1])))
    G.log(f"   flags 0x{flags:x}")
    assert flags & (L.WAIT_ATTN_LOADER | L.WAIT_ATTN_COMPUTE) and not flags & L.WAIT_TOKEN
    # default limit: nothing reported, the reference output again
    assert torch.equal(G.dr().sparse_attn(q, k, v, cand, kept), ref)
    assert torch.equal(G.dr().attn(q[:, :1], k[:, :1], v[:, :1]), ref_d)
    assert G.dr().wait_report() == 0


def test_token_selection_waits_report_give_ups():
    import torch
    G.log("[wait] token selection under a one-poll limit")
    from block_sparse_attention_candidates_amd import _lib as L
    name = "wan13b_480p"
    q, k, _ = G.device_qkv(name)
    q, k = (x[:, :2].contiguous() for x in (q, k))
    cand = G.candidates(name)
    pr = workloads.TOKEN_PRESETS["mid"]
    ref = G.dr().token_select(q, k, cand, pr["tau_near"], pr["tau_far"])
    flags = _limited(lambda: G.dr().token_select(q, k, cand, pr["tau_near"], pr["tau_far"]))
    G.log(f"   flags 0x{flags:x}")
    assert flags == L.WAIT_TOKEN
    again = G.dr().token_select(q, k, cand, pr["tau_near"], pr["tau_far"])
    assert torch.equal(again.kept_cnt, ref.kept_cnt) and torch.equal(again.kept_col, ref.kept_col)
    assert G.dr().wait_report() == 0
