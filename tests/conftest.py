import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_addoption(parser):
    parser.addoption("--run-slow", action="store_true", default=False,
                     help="also run the long exhaustive CPU pins")


def pytest_collection_modifyitems(config, items):
    if config.getoption("--run-slow"):
        return
    skip = pytest.mark.skip(reason="long exhaustive pin; run with --run-slow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long CPU test")


def _ensure_host_builds():
    """Build the CPU-side helpers only when nothing is built yet."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not os.path.exists(synth.HOST_LIB):
        synth.build(device=False)


_ensure_host_builds()
