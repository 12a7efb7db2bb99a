import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-shape test (minutes of host work)")


@pytest.fixture(scope="session")
def lib():
    """The built HIP library through its Python binding; GPU tests only."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import audio_video_diffusion_block_amd as h3
    return h3
