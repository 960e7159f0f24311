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


class _AOptions:
    """Plan overrides of the A update through the library's debug hook
    (seacells_debug_set_a_options); merged across calls, reset after the test."""

    def __init__(self):
        self.cur = {}

    def _apply(self):
        import sparse_archetypal_analysis_amd as saa
        saa.seacells_debug_set_a_options(**self.cur)

    def set(self, **kw):
        self.cur.update(kw)
        self._apply()

    def clear(self, *names):
        for nm in names:
            self.cur.pop(nm, None)
        self._apply()


@pytest.fixture
def a_options():
    opts = _AOptions()
    yield opts
    opts.cur = {}
    opts._apply()
