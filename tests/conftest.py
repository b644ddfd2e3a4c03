import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line(
        "markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu():
    """Session fixture for GPU tests: fails (never skips) without a GPU, so a
    GPU run cannot pass by silently skipping its parity tests."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import blockwise_scaled_fp8_amd as fp8
    fp8.load_library()
    return torch.device("cuda", 0)
