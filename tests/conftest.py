import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: full-size parity case (minutes of CPU oracle time)")


def golden(name):
    """Rows of a whitespace-separated fixture under tests/golden, comments stripped."""
    rows = []
    with open(os.path.join(ROOT, "tests", "golden", name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append(line.split())
    return rows


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP library on a GPU; fails loudly when it is missing on a GPU machine."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_sparse_spatio_amd as vsa
    vsa.load()  # raises if libvsa.so is missing
    return vsa
