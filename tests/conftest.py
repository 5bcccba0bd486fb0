import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built libpda.so")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding, loaded once; skips nothing: a GPU test without the
    built library or a GPU fails loudly."""
    import torch
    assert torch.cuda.is_available(), "GPU test run without a visible GPU"
    import decode_attention_fp8_write_amd as pda
    pda.load()
    return pda
