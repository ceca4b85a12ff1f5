import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libwallattn")


@pytest.fixture(autouse=True)
def _announce(request):
    """Name each test on stderr before it runs, so a run that dies mid-test says where."""
    sys.__stderr__.write(f"\n[start] {request.node.nodeid}\n")
    sys.__stderr__.flush()
    yield
