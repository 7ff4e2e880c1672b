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
    """The HIP library, loaded; skips nothing: a GPU test without the
    library or without a GPU fails loudly."""
    import torch
    import token_early_exit_amd as tee
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    lib = tee.load()
    return tee
