import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: longer CPU test")


def pytest_collection_modifyitems(config, items):
    # Print the test id before each GPU test runs so a failing box still names the case.
    pass


@pytest.fixture(autouse=True)
def _announce(request):
    if request.node.get_closest_marker("gpu") is None:
        yield
        return
    print("\n[gpu-test] %s" % request.node.nodeid, flush=True)
    # every output, state and workspace buffer the binding allocates starts
    # as NaN, so an element a kernel leaves unwritten cannot pass as a stale
    # correct value
    from gated_deltanet_recurrence_frame_amd import binding
    old = binding.POISON
    binding.POISON = True
    try:
        yield
    finally:
        binding.POISON = old
