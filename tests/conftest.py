import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large inputs (minutes on the CPU)")


def _flush_print(msg):
    print(msg, flush=True)


@pytest.fixture(autouse=True)
def _announce(request):
    # GPU steps print the case they run before touching the device, so that a
    # run that ends the process still names the case that was running.
    if request.node.get_closest_marker("gpu") is not None:
        _flush_print(f"\n[gpu-case] {request.node.nodeid}")
    yield
