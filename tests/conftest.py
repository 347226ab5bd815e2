import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def pytest_collection_modifyitems(config, items):
    try:
        import torch
        have_gpu = torch.cuda.is_available()
    except Exception:
        have_gpu = False
    if have_gpu:
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)


@pytest.fixture(scope="session")
def orc():
    from oracle import oracle
    src = os.environ.get("FP8Q_ORACLE_SOURCE")
    if src:
        # the oracle built from another source file: tests/test_oracle_mutants.py runs the oracle's
        # pins against copies of oracle.c with one planted mistake each
        oracle._SRC = src
        oracle._LIB_PATH = os.path.splitext(src)[0] + ".so"
    oracle.lib()
    return oracle
