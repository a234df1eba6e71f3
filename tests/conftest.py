import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libopq")
    config.addinivalue_line("markers", "slow: a CPU test that takes more than a few seconds")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded C-ABI binding; fails loudly when the library is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("gpu test selected but no GPU is visible")
    from w4a16_linear_amd import opq
    opq.load()
    return opq
