import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs a real MI355X (runs through the HIP library)")
    config.addinivalue_line("markers", "slow: full-size workload, minutes of oracle time")


@pytest.fixture(scope="session", autouse=True)
def _oracle_built():
    from oracle import build as ob
    if not os.path.exists(ob.LIB) or os.path.getmtime(ob.LIB) < os.path.getmtime(ob.SRC):
        ob.build_oracle()
    yield


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The GPU tests' normwise errors against the oracle (tolerances 2e-2 on o, 1e-2 on the
    state), one line per checked case, so that a passing run still shows its margins."""
    try:
        from tests.gpu_util import REPORT
    except Exception:   # the GPU helpers were never imported (CPU-only run)
        return
    if REPORT:
        terminalreporter.section("parity errors against the fp64 oracle (o, state)")
        for line in REPORT:
            terminalreporter.write_line(line)
