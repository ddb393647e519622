import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running check")


@pytest.fixture(scope="session")
def gpu_lib():
    """The GPU library, loaded (never built) for GPU tests; fails loudly if missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import dense_gemm_12_amd as mg
    mg.load()
    return mg
