import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libdflash2")
    config.addinivalue_line("markers", "slow: long CPU test")


def pytest_collection_modifyitems(config, items):
    # Only skip GPU tests when no GPU is present; never silently pass them.
    try:
        import torch
        has_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        has_gpu = False
    if has_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


def pytest_terminal_summary(terminalreporter, exitstatus, config):
    """Reports how many walk steps and verify requests the parity checks compared with
    the oracle, and how many of their decisions the oracle itself placed within the
    1e-5 band of a tie or a boundary (near ties and band differences)."""
    try:
        import parity_util
    except Exception:  # pragma: no cover
        return
    c = parity_util.COUNTS
    if not (c["walk_steps"] or c["verify_requests"]):
        return
    terminalreporter.write_line(
        "parity decisions: walk steps {walk_steps} (near ties {walk_near_ties}, in band {walk_band}); "
        "verify requests {verify_requests} (in band {verify_band})".format(**c))
    import json
    out_dir = os.path.join(ROOT, os.environ.get("DFLASH2_OUT_DIR", "gpurun_out"))
    try:
        os.makedirs(out_dir, exist_ok=True)
        with open(os.path.join(out_dir, "parity_counts.json"), "w") as f:
            json.dump(c, f)
    except OSError:  # pragma: no cover
        pass
