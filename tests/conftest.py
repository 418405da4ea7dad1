import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libccq.so")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; GPU tests fail loudly (not skip) when it is missing."""
    import torch
    from curvature_conditioned_query_amd import load_library
    assert torch.cuda.is_available(), "gpu-marked test run without a GPU"
    return load_library()
