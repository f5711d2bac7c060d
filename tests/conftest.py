import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle.build()
    return oracle


@pytest.fixture(scope="session")
def mx():
    """The HIP library binding, built in-tree first if it is missing; GPU tests only."""
    import torch
    from block_scaled_precision_act_amd import mxgemm
    if not os.path.exists(mxgemm.LIB_PATH):
        from block_scaled_precision_act_amd import build
        build.build(verbose=False)
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    mxgemm.lib()
    return mxgemm
