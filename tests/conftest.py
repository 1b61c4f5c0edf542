import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950); calls the HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Print the parity report lines the GPU tests recorded (near-tie counts
    of the sampled verify and the gate, tolerance allowances used), so that
    they survive a quiet (-q) run."""
    from tests.gpu_util import REPORT
    if REPORT:
        terminalreporter.section("parity report")
        for line in REPORT:
            terminalreporter.write_line(line)
