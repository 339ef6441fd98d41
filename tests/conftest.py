import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def have_gpu():
    import torch
    return torch.cuda.is_available()


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The parity tallies of the run (draws, near-ties, draws within 1e-5 of an edge,
    hard mismatches), one line per check that reported one."""
    try:
        from parity_util import REPORT
    except ImportError:
        return
    if not REPORT:
        return
    terminalreporter.write_sep("-", "parity tallies (GPU vs fp64 oracle)")
    for name, t in REPORT:
        terminalreporter.write_line(f"{name}: {t}")
