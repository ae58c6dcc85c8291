import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(autouse=True)
def _announce_gpu_case(request):
    """Name each GPU case before it runs (stderr and an optional progress file),
    so a run that ends abruptly still shows which case was on the GPU."""
    if request.node.get_closest_marker("gpu") is not None:
        line = f"[gpu-case] {request.node.nodeid}\n"
        sys.stderr.write(line)
        sys.stderr.flush()
        path = os.environ.get("NPA_TEST_PROGRESS")
        if path:
            with open(path, "a") as f:
                f.write(line)
    yield
