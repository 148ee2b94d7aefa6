import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _device_error_word(request):
    """GPU tests: the device error word (hcs_device_errors) must be clear after the test; a test
    that provokes an error on purpose reads and clears it itself."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    import hybrid_compressed_sparse_amd as hcs
    bits = hcs.device_errors(clear=True)
    assert bits == 0, f"device error word 0x{bits:x} set during {request.node.name}"
