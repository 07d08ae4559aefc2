import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu():
    """The HIP binding on cuda:0; the test fails loudly if the library is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("a gpu-marked test ran without a visible GPU")
    from quantized_moe_expert_fp32_amd import moe

    return moe
