import os
import sys
from pathlib import Path

import pytest

ROOT = Path(__file__).resolve().parent.parent
if str(ROOT) not in sys.path:
    sys.path.insert(0, str(ROOT))


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


def pytest_collection_modifyitems(config, items):
    """GPU tests skip when no GPU is visible, unless TG_REQUIRE_GPU=1 asks them to fail."""
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:  # pragma: no cover
        have_gpu = False
    if have_gpu or os.environ.get("TG_REQUIRE_GPU") == "1":
        return
    skip = pytest.mark.skip(reason="no GPU visible (set TG_REQUIRE_GPU=1 to fail instead)")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
