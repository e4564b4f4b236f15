import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; the parity tests proper")


@pytest.fixture(scope="session")
def gpu():
    """The HIP library bound to cuda:0.  Fails (does not skip) without a GPU:
    a GPU test that silently skipped would hide a missing native path."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    from w4a4_rotated_bit_amd import binding
    binding.load()
    return binding
