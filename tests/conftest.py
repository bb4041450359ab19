import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """The worst row-relative error each floating-point comparison reached,
    against its tolerance (the margin to the bar), in the order they ran."""
    from tests.parity import MARGINS
    if not MARGINS:
        return
    tr = terminalreporter
    tr.section("parity margins: worst row-relative error / tolerance")
    for what, worst, tol in MARGINS:
        tr.write_line(f"{worst:10.3e} / {tol:.0e}  {what}")
