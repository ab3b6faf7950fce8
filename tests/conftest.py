import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test (large workload)")


_plans = {}


@pytest.fixture(scope="session")
def workload_plan():
    """Cached (workload, positions, oracle plan) per workload key."""
    import oracle
    import workloads as W

    def get(k):
        if k not in _plans:
            w = W.WORKLOADS[k]
            x = W.positions(w)
            _plans[k] = (w, x, oracle.OraclePlan(x, **w.params()))
        return _plans[k]

    return get


@pytest.fixture(autouse=True)
def _announce(request):
    """Name every test on the real stderr before it runs (GPU runs stay legible
    even when a box ends mid-test)."""
    if request.node.get_closest_marker("gpu") is not None:
        sys.__stderr__.write(f"\n[start] {request.node.nodeid}\n")
        sys.__stderr__.flush()
    yield
