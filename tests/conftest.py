import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_terminal_summary(terminalreporter):
    """Repeat the parity tallies (exact / near-tie / near-threshold counts)
    collected by tests/parity.py, so that they show in a -q run."""
    mod = sys.modules.get("tests.parity")
    lines = getattr(mod, "SUMMARY", None)
    if lines:
        terminalreporter.write_sep("-", "parity tallies")
        for line in lines:
            terminalreporter.write_line(line)
