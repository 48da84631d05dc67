import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover - torch is part of the image
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


# The library honours its tuning and cross-check overrides (FP8W8A8_FORCE_PATH
# and the like, which several GPU tests set) only with this switch, read once
# when the library first looks; production processes never set it.
os.environ.setdefault("FP8W8A8_TEST_HOOKS", "1")


def pytest_sessionfinish(session, exitstatus):
    """With FP8W8A8_PARITY_REPORT=<path>, write every output comparison of
    the run (oracle.check.REPORT_LOG: largest error over the row RMS, the
    floor that comparison needs) to <path> as JSON."""
    path = os.environ.get("FP8W8A8_PARITY_REPORT")
    if not path:
        return
    import json
    try:
        from oracle.check import REPORT_LOG
    except Exception:  # pragma: no cover - the oracle is part of the repo
        return
    os.makedirs(os.path.dirname(os.path.abspath(path)), exist_ok=True)
    with open(path, "w") as f:
        json.dump(REPORT_LOG, f, indent=0)
