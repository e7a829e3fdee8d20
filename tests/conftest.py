import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP path")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0; skips when no GPU is visible, fails when the
    built library is missing (never falls back to anything else)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_scaled_fp8_gemm_amd as fbg
    fbg.load()  # raises if the HIP library is not built
    return fbg
