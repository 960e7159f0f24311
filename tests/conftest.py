import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: larger CPU cases")


def pytest_collection_modifyitems(config, items):
    # Print the case name before every GPU test, flushed, so a run that ends
    # the process still names what was running.
    for item in items:
        if item.get_closest_marker("gpu") is not None:
            item.add_marker(pytest.mark.usefixtures("_announce_gpu_case"))


@pytest.fixture
def _announce_gpu_case(request):
    print("\n[gpu-case] %s" % request.node.nodeid, flush=True)
    sys.stdout.flush()
    yield
