import json
import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def repo_root():
    return ROOT


@pytest.fixture(autouse=True)
def _parity_case(request):
    """Name the parity-report entry after the running test (tests may refine it)."""
    mod = sys.modules.get("tests.test_gpu_attention")
    if mod is not None:
        mod.set_case(request.node.nodeid.split("::", 1)[-1])
    yield


def pytest_sessionfinish(session, exitstatus):
    """With CM_PARITY_REPORT=path, write every comparison's worst excess of
    |got - exact| over the plain 2e-2 (negative = margin), per case and
    output, as JSON."""
    path = os.environ.get("CM_PARITY_REPORT")
    mod = sys.modules.get("tests.test_gpu_attention")
    if not path or mod is None or not mod.PARITY_REPORT:
        return
    rep = mod.PARITY_REPORT
    worst = {}
    for case, rec in rep.items():
        for name, x in rec.items():
            if name not in worst or x > worst[name][0]:
                worst[name] = (x, case)
    with open(path, "w") as f:
        json.dump({"atol": mod.ATOL, "worst": worst, "cases": rep}, f, indent=1, sort_keys=True)
