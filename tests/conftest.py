import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(autouse=True)
def _name_the_case(request):
    """Print each test's id before it runs, unbuffered, so that a run cut
    short on the GPU still shows which case was in flight."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[case] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
