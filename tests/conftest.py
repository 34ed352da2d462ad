"""Shared pytest setup.

Tests marked ``gpu`` run the HIP library through its C ABI on an MI355X; they
fail (never skip) when no GPU is visible, so a GPU run cannot pass vacuously.
Everything else runs on the CPU: the oracle against its pins, the input
generators, and the host side of the C ABI.
"""
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X; runs the HIP kernels through the C ABI")


@pytest.fixture(scope="session")
def gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but no GPU is visible")
    import paged_kv_cache_243_amd as pkv  # raises if the HIP library is missing
    return pkv
