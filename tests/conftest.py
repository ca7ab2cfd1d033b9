import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    # Build the CPU-side libraries only when nothing is built yet.
    import oracle
    import synth
    for mod in (oracle, synth):
        so = mod._SO
        if not os.path.exists(so):
            mod.build()


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library binding; fails loudly when the library or the GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test started without a visible GPU")
    import quantized_q4_q8_amd as qk
    qk.load()
    return qk
