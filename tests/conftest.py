import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large-size case")


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on cuda:0; fails loudly when it is not built."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU visible")
    import block_draft_model_dspark_amd as dsp
    dsp.load_library()
    return dsp
