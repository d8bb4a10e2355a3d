import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path through the C-ABI")


def pytest_collection_modifyitems(config, items):
    # GPU tests are skipped, not failed, when no GPU is present and -m gpu was not asked for.
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# Lines the whole-output parity tests record (count compared, largest error); printed at the
# end of the session so they show under -q as well.
PARITY_REPORT = []


def pytest_terminal_summary(terminalreporter):
    if PARITY_REPORT:
        terminalreporter.section("whole-output parity against the fp64 oracle")
        for line in PARITY_REPORT:
            terminalreporter.write_line(line)
