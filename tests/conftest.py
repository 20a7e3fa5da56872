import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library")
    config.addinivalue_line("markers", "slow: long-running case")


@pytest.fixture(scope="session")
def gpu():
    """The GPU device; GPU tests fail loudly (not skip) when none is present."""
    import torch
    assert torch.cuda.is_available(), "GPU test collected on a machine without a GPU"
    return torch.device("cuda:0")
