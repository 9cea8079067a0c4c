"""Shared fixtures.  GPU tests are marked ``gpu`` (registered in pytest.ini)."""

import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


@pytest.fixture(scope="session")
def dev():
    """cuda:0 with the HIP library loaded; skips only where no GPU exists."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU on this host")
    from vocab_log_softmax_amd import rlk
    rlk.load_library()          # raises if librlk.so is missing: no silent fallback
    return torch.device("cuda:0")


@pytest.fixture(scope="session")
def orc():
    import oracle
    o = oracle.get()
    o.set_threads(min(16, len(os.sched_getaffinity(0))))
    return o
