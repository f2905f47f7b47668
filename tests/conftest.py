"""Shared pytest configuration.

Tests marked ``gpu`` need a gfx950 device and the built ``libfa355.so``; all
other tests run on the CPU.
"""

import pytest


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP library through its C ABI")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails loudly (never skips) if it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    import io_aware_softmax_06_amd as fa
    fa.load()
    return fa
