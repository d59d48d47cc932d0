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
    """The HIP library, on a machine with a GPU.  Fails (never skips) when the
    library is missing, so a GPU run cannot pass on a silent fallback."""
    import torch
    from exact_attention_forward_06_amd import _lib
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    return _lib.load()
