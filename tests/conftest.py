import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libkda.so")


@pytest.fixture(scope="session")
def oracle_c():
    """The C fp64 oracle (built on first use)."""
    from oracle import kda_oracle
    kda_oracle.lib()
    return kda_oracle


def pytest_collection_modifyitems(config, items):
    """GPU tests need a GPU; without one (e.g. the CPU container) they are
    skipped.  With a GPU present a missing libkda.so fails them loudly."""
    if not any("gpu" in item.keywords for item in items):
        return
    import torch
    if torch.cuda.is_available():
        return
    skip = pytest.mark.skip(reason="no GPU in this process")
    for item in items:
        if "gpu" in item.keywords:
            item.add_marker(skip)
