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
    """The HIP library, on a GPU. Fails loudly (no fallback) if it is missing."""
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test collected without a visible GPU")
    from bit_nf4_quantized_18_amd import binding

    binding.load()  # raises if libqlora_nf4.so is absent
    return binding
