import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libdsa.so")
    config.addinivalue_line("markers", "slow: long-running (large workload) test")


def pytest_collection_modifyitems(config, items):
    # GPU tests at the end, large ones last, so a quick failure shows first;
    # the no-allocation entry point's tests after everything else, so that
    # they run on a GPU whose scratch array earlier tests have already used.
    def key(item):
        return (1 if item.module.__name__.endswith("test_zz_no_alloc") else 0,
                1 if item.get_closest_marker("gpu") else 0,
                1 if item.get_closest_marker("slow") else 0)
    items.sort(key=key)


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    return torch.cuda.is_available()


def pytest_sessionfinish(session, exitstatus):
    # DSA_PARITY_RECORD=<file>: write the boundary-swap counts of every
    # index comparison this run made (a markdown table)
    path = os.environ.get("DSA_PARITY_RECORD")
    if not path:
        return
    import parity
    if parity.SWAP_LOG:
        parity.write_swap_record(path)
