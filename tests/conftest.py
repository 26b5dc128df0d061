"""Shared pytest configuration: the ``gpu`` marker and lazily built native libraries."""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def gpu_device():
    """The first HIP device; skips nothing: a gpu-marked test without a GPU is an error."""
    import torch

    if not torch.cuda.is_available():
        raise RuntimeError("gpu-marked test run without a visible GPU")
    return torch.device("cuda:0")
