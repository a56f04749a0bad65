import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
TESTS = os.path.dirname(os.path.abspath(__file__))
for p in (ROOT, TESTS):
    if p not in sys.path:
        sys.path.insert(0, p)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case on the terminal before it touches the device (run with -s)."""
    if request.node.get_closest_marker("gpu") is not None:
        print(f"\n[gpu case] {request.node.nodeid}", flush=True)
    yield
