import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

GOLDEN = os.path.join(ROOT, "tests", "golden")


def pytest_addoption(parser):
    parser.addoption("--runslow", action="store_true", default=False,
                     help="also run tests marked slow (long exhaustive CPU sweeps)")


def pytest_collection_modifyitems(config, items):
    if config.getoption("--runslow"):
        return
    skip = pytest.mark.skip(reason="slow sweep: run with --runslow")
    for item in items:
        if "slow" in item.keywords:
            item.add_marker(skip)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: exhaustive CPU sweep taking minutes (runs only with --runslow)")


def read_golden(name):
    """Rows of a whitespace-separated golden fixture, comments stripped."""
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def orc():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def gpu():
    """The HIP library on cuda:0.  Skips only when no GPU is visible; with a
    GPU the library must load (it is built first if missing, and a failed
    build fails the test loudly: there is no other path)."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible (run with -m gpu on an MI355X)")
    import block_scaled_precision_mxfp8_amd as mxq
    mxq.load()  # raises if libmxq.so cannot be built or loaded
    return mxq
