import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; calls the HIP path")


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded HIP library; fails loudly if it or the GPU is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected on a machine without a GPU")
    import row_wise_backward_amd as rwb

    return rwb


@pytest.fixture(autouse=True)
def _sentinel_bands(request):
    """After every GPU test: the sentinel bands around every 2-D input and
    output buffer, and the gaps between the rows of padded layouts, are
    unchanged."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import gpu_util

    bad = gpu_util.guards_broken()
    assert not bad, f"write outside a buffer: {bad}"
