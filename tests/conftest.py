import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _gpu_available() -> bool:
    try:
        import torch
    except Exception:
        return False
    return bool(torch.cuda.is_available())


def pytest_collection_modifyitems(config, items):
    if _gpu_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    # parity totals of the GPU comparisons run in this session (see gpu_helpers.TOTALS)
    helpers = sys.modules.get("gpu_helpers")
    totals = getattr(helpers, "TOTALS", None)
    if totals and totals["comparisons"]:
        terminalreporter.write_line(
            "parity totals: {comparisons} comparisons, {sequences} sequences, {exact} exact, {flips} near-tie flips, "
            "{failures} failures, largest relative probability error {max_prob_rel_err:.3e}".format(**totals))
