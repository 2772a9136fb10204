"""Shared pytest configuration.

Tests marked ``gpu`` need a ROCm GPU and the built HIP library; everything
else runs on the CPU.
"""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a ROCm GPU and the HIP library")
    config.addinivalue_line("markers", "slow: large CPU-only case")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def cuda():
    """The GPU device.  Skips only on a machine without a ROCm device node;
    a machine that has one but cannot use it fails loudly."""
    if not gpu_available():
        if os.path.exists("/dev/kfd"):
            pytest.fail("a ROCm device node exists but torch sees no GPU")
        pytest.skip("no GPU on this machine")
    import torch
    return torch.device("cuda:0")
