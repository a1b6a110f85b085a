import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library, loaded; fails loudly (never skips, never falls back)
    when it is missing or no GPU is visible."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import blockwise_scaled_fp8_amd as bfp8
    bfp8.load()  # raises if libbfp8.so is absent
    return bfp8
