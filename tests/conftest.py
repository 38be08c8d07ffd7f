import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: long-running CPU test")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library through its Python binding; skips cleanly without a GPU."""
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import nvfp4_w4a4_block_quantize_amd as nv

    nv.load_library()  # raises if the HIP library is missing: no silent fallback
    return nv
