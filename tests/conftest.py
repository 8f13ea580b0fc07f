import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; parity tests through the C ABI")


@pytest.fixture(scope="session")
def golden_dir():
    return os.path.join(ROOT, "tests", "golden")


@pytest.fixture(autouse=True)
def _no_expired_device_waits(request):
    """After every GPU test: no bounded wait inside a kernel ran out (an
    expired wait lets the kernel finish but makes its outputs unreliable)."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch
    if not torch.cuda.is_available():
        return
    from bit_ternary_weight_amd import binding
    n = binding.device_errors(reset=True)
    assert n == 0, f"{n} bounded waits expired on the device during this test"
