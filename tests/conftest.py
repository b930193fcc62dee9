import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def dynrad_lib():
    """The built C-ABI library (built once if missing)."""
    from block_sparse_attention_candidates_amd import _lib
    if not os.path.exists(_lib.LIB_PATH):
        from block_sparse_attention_candidates_amd import build
        build.build()
    return _lib.lib()


@pytest.fixture(autouse=True)
def _no_wait_gave_up(request):
    """After every GPU test: no bounded wait of a ring kernel gave up
    (dr_wait_report reads and clears the device's flags; raises if any)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    import block_sparse_attention_candidates_amd as dr
    dr.set_wait_limit(0)
    assert dr.wait_report() == 0
