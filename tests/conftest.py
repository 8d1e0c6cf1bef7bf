import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def oracle():
    import oracle as o
    o.build(force=False)
    return o


def pytest_sessionfinish(session, exitstatus):
    """Keeps the routing tie-band counts of a GPU run (how many rows a near
    tie let differ, by stage) as tie_band.json in the directory that
    HGA_TEST_REPORT_DIR names, when it is set and exists."""
    gc = sys.modules.get("gpu_common")
    out = os.environ.get("HGA_TEST_REPORT_DIR", "")
    if gc is None or not gc.TIE_LOG or not out or not os.path.isdir(out):
        return
    import json
    with open(os.path.join(out, "tie_band.json"), "w") as f:
        json.dump(gc.TIE_LOG, f, indent=1)
