import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def read_table(name):
    """Rows of a whitespace table under tests/golden/, comments skipped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            rows.append(line.replace("->", " ").split())
    return rows


@pytest.fixture(scope="session")
def table():
    return read_table


@pytest.fixture(autouse=True)
def _device_status_clean(request):
    """After every GPU test: no batch kernel recorded a barrier wait that gave
    up, nor (debug build) a failed device check.  Tests that force one read
    and clear the record themselves."""
    yield
    if request.node.get_closest_marker("gpu") is None:
        return
    import async_tensor_tile_amd as att
    if att._lib is None:
        return
    att.tile_device_status(0)
