"""Shared pytest configuration.

Tests marked ``gpu`` need a real MI355X and the built HIP library; everything
else runs on the CPU.  The ``gpu`` marker is registered here so that
``pytest -m gpu`` / ``-m "not gpu"`` select cleanly.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an AMD GPU (gfx950) and the built HIP library")


@pytest.fixture(scope="session")
def gpu_device():
    """Skip-free GPU fixture: a gpu-marked test on a machine without a GPU fails loudly."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("gpu-marked test run without a visible GPU")
    return torch.device("cuda:0")
