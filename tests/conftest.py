import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle cases that take tens of seconds")


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Report every pivot comparison that stopped at an fp64/fp32 near tie."""
    helpers = sys.modules.get("_helpers")
    if helpers is None:   # no parity test ran
        return
    NEAR_TIE_EXITS = helpers.NEAR_TIE_EXITS
    terminalreporter.write_line(f"pivot comparisons stopped at a near tie: {len(NEAR_TIE_EXITS)}")
    for ctx, i, margin in NEAR_TIE_EXITS:
        terminalreporter.write_line(f"  {ctx}: draw {i}, margin {margin:.3e}")
