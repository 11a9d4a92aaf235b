import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def dev():
    """The GPU and the built HIP library; tests marked gpu fail loudly when the
    library is missing instead of falling back to anything."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import moe_grouped_gemm_fp8_amd as fg8
    fg8._lib.lib()
    return torch.device("cuda:0")
