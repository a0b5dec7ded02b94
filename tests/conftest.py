import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU check")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library and a CUDA device, or a hard failure on a machine with a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this container")
    import fp8_scaled_gemm_amd as fp8g
    fp8g.load()          # raises if the built library is missing
    return fp8g
