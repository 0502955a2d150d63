import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: large shapes; still part of the default suite")


@pytest.fixture(autouse=True)
def _gpu_test_requirements(request):
    """A GPU test fails (never skips) when there is no GPU or the HIP library does not load."""
    if request.node.get_closest_marker("gpu") is None:
        return
    import torch

    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a GPU")
    import bit_quantized_finetuning_amd.qlora  # noqa: F401  (raises ImportError when libqlora.so is missing)
