import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size case (seconds to minutes)")


def pytest_collection_modifyitems(config, items):
    have_gpu = False
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        pass
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in items:
        if "gpu" in it.keywords:
            it.add_marker(skip)


def pytest_terminal_summary(terminalreporter):
    """Print the near-tie report of the routing comparisons (tokens whose
    top-K margin is within the tie band, and how many of them the GPU chose
    differently from the float64 oracle)."""
    try:
        from helpers import NEAR_TIE_REPORT
    except Exception:
        return
    if NEAR_TIE_REPORT:
        terminalreporter.write_sep("-", "near-tie tokens")
        for line in NEAR_TIE_REPORT:
            terminalreporter.write_line(line)
