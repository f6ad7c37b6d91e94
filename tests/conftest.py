import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


def _ensure_host_libs():
    """Build the gcc-compiled helpers (generator, oracle) if they are absent."""
    import oracle
    import synth

    if not os.path.exists(os.path.join(ROOT, "synth", "libsynth.so")):
        synth.build()
    if not os.path.exists(os.path.join(ROOT, "oracle", "liboracle.so")):
        oracle.build()


_ensure_host_libs()


@pytest.fixture(scope="session")
def gpu_ready():
    import torch

    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return torch.device("cuda:0")
