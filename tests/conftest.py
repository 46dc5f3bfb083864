import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: long-running CPU test")


def _ensure_cpu_libs():
    """Build the host-only libraries if nothing is built yet (gcc, a second or two)."""
    import oracle
    import synth
    if not os.path.exists(oracle.LIB):
        oracle.build()
    if not os.path.exists(synth.CPU_LIB):
        synth.build()


_ensure_cpu_libs()


@pytest.fixture(scope="session")
def gpu_available():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return True
