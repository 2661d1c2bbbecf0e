import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running GPU case at a full workload size")


# GPU tests announce themselves (flushed) before they run, so that a run that ends the
# process still names the case that was running.
@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    if request.node.get_closest_marker("gpu") is not None:
        sys.stdout.write("\n[gpu case] %s\n" % request.node.nodeid)
        sys.stdout.flush()
    yield
