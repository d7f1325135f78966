import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def dsa_gpu():
    """The HIP library bound through ctypes, on cuda:0.  Fails loudly when the
    library is missing; skips only when no GPU is present at all."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU in this process")
    import long_context_lightning_amd as lcl
    lcl.load()  # raises if libdsa.so is missing or fails to load
    return lcl
