import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def pytest_collection_modifyitems(config, items):
    # Collect the GPU parity tests in file order; nothing else to reorder.
    pass


def pytest_runtest_logfinish(nodeid, location):
    # Progress reaches a pipe after every test, not only at the end of each line of
    # results (stdout is block-buffered there, and the full-size tests run for minutes).
    sys.stdout.flush()


@pytest.fixture(scope="session")
def dg_ctx():
    """One libdg context on cuda:0 for the GPU tests (fails loudly without a GPU)."""
    import torch

    import block_ar_canvas_amd as dg

    assert torch.cuda.is_available(), "GPU tests need an MI355X"
    ctx = dg.Context(0)
    yield ctx
    ctx.close()
