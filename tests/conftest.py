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
    """The HIP library, loaded through its Python binding.  GPU tests use this;
    a missing or unloadable library is an error, never a skip or a fallback."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import prefix_shared_tree_packed_amd as pst
    pst.load()
    return pst
