import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu():
    """The loaded HIP library on cuda:0; GPU tests fail loudly if it is missing."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a GPU"
    from tile_pipelined_gemm_amd import mk
    mk.load()
    return mk
