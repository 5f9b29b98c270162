"""Test configuration: the `gpu` marker and import paths.

Tests marked ``gpu`` need a ROCm device and call the HIP library through its C
ABI; everything else runs on the CPU (oracle pins, host logic, ABI loading
and argument validation).
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def oracle_mod():
    import oracle
    return oracle
