import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

# The host AddressSanitizer run of the ABI tests (tests/test_abi_asan.py)
# points the binding at the sanitized build of the library.
if os.environ.get("MIATTN_TEST_LIBRARY"):
    import exact_attention_37_amd as _mi
    _mi.library_path = os.environ["MIATTN_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libmiattn")
    config.addinivalue_line("markers", "slow: long-running (full-size workloads)")


def pytest_collection_modifyitems(config, items):
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU visible")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
