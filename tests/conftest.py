import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (MI355X) and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The GPU tests never skip silently: without a device they fail."""
    import torch
    assert torch.cuda.is_available(), "gpu-marked test run without a visible GPU"
    return torch.device("cuda:0")
