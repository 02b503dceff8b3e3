import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case")


def pytest_collection_modifyitems(config, items):
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """One line of error statistics per parity check that recorded them (full-size workloads,
    the precision measurement), so they appear in the run's tail."""
    try:
        from tests.tolerance import summary_lines
    except Exception:
        return
    lines = summary_lines()
    if lines:
        terminalreporter.write_sep("-", "parity statistics")
        for line in lines:
            terminalreporter.write_line(line)
