import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_terminal_summary(terminalreporter):
    """The GPU parity cases' near-tie counts (tests/parity_log.py), printed even under -q."""
    import parity_log
    lines = parity_log.summary_lines()
    if lines:
        terminalreporter.section("parity: requests compared, near-ties (oracle margin <= 1e-6)")
        for ln in lines:
            terminalreporter.write_line(ln)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")
