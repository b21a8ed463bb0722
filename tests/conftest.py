import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU case")


def pytest_collection_modifyitems(config, items):
    # GPU tests print the case they run before touching the device, so a
    # failure that ends the process still names its case.
    for item in items:
        if item.get_closest_marker("gpu") is not None:
            item.add_marker(pytest.mark.usefixtures("_announce_case"))


@pytest.fixture
def _announce_case(request):
    print(f"\n[case] {request.node.nodeid}", flush=True)
    yield
