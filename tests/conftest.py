import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--run-slow", action="store_true", default=False,
                     help="also run tests marked slow (full-size acceptance checks "
                          "whose fp64 oracle side takes many minutes)")


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line(
        "markers", "slow: full-size acceptance check (minutes of oracle time); runs "
                   "with --run-slow or RF_RUN_SLOW=1")


def pytest_collection_modifyitems(config, items):
    run_slow = config.getoption("--run-slow") or os.environ.get("RF_RUN_SLOW") == "1"
    if not run_slow:
        skip_slow = pytest.mark.skip(reason="slow acceptance check: --run-slow")
        for it in items:
            if "slow" in it.keywords:
                it.add_marker(skip_slow)
    gpu_items = [it for it in items if "gpu" in it.keywords]
    if not gpu_items:
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this environment")
    for it in gpu_items:
        it.add_marker(skip)
