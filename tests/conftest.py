import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    """Skip GPU tests cleanly when no GPU is visible (the CPU suite runs everywhere)."""
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Worst error / bound ratio of each parity check, per test (filled by the GPU
# parity tests, printed at the end of the run).
PARITY_RATIOS: dict = {}


def pytest_terminal_summary(terminalreporter):
    if not PARITY_RATIOS:
        return
    tr = terminalreporter
    tr.section("worst error / bound per parity test")
    for test, checks in PARITY_RATIOS.items():
        worst = max(checks.values())
        detail = ", ".join(f"{k} {v:.3f}" for k, v in checks.items())
        tr.write_line(f"{worst:.3f}  {test}: {detail}")
    overall = max(max(c.values()) for c in PARITY_RATIOS.values())
    tr.write_line(f"overall worst error / bound: {overall:.3f}")
