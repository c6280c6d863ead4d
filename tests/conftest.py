import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) and the built HIP library")
    config.addinivalue_line("markers", "slow: large CPU oracle runs")


@pytest.fixture(scope="session")
def lib():
    """The HIP library's Python binding, with the device checked."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import linear_attention_lact_amd as ttt
    ttt.load()  # raises if the shared library is missing
    return ttt
