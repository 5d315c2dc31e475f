import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


@pytest.fixture(scope="session")
def orc():
    import oracle
    oracle._load()
    return oracle


@pytest.fixture(autouse=True)
def _guarded_outputs(request, monkeypatch):
    """GPU tests: every buffer the binding allocates carries canaries,
    checked once the test's kernels have finished."""
    if request.node.get_closest_marker("gpu") is None:
        yield None
        return
    import torch
    import quantized_gemm_q4_amd as q4
    from parity import GuardedAllocator
    guard = GuardedAllocator()
    monkeypatch.setattr(q4, "_empty", guard)
    yield guard
    torch.cuda.synchronize()
    guard.check()


def pytest_sessionfinish(session, exitstatus):
    """Q4_MARGINS_OUT=<file>: write the accuracy margin of every GEMM parity
    check (worst |Y - Y_ref| / B and relative L2) as JSON."""
    path = os.environ.get("Q4_MARGINS_OUT")
    if not path:
        return
    import json
    from parity import MARGINS
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(MARGINS, f, indent=0)
