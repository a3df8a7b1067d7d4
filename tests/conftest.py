import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP path's Python binding, on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but torch sees no GPU")
    import rank_gemm_amd
    return rank_gemm_amd
