import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of oracle work)")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library on cuda:0; fails (not skips) if the GPU or the
    library is missing, so a GPU run can never pass without native code."""
    import torch
    assert torch.cuda.is_available(), "gpu test run without a visible GPU"
    from block_scaled_precision_bsgemm_amd import lib
    return lib.load()
