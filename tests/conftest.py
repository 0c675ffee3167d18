import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
for _p in (ROOT, os.path.join(ROOT, "tests")):
    if _p not in sys.path:
        sys.path.insert(0, _p)


def gpu_available():
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")
    config.addinivalue_line("markers", "slow: oracle work of more than a few seconds")


@pytest.fixture(scope="session")
def golden():
    import json

    def load(name):
        with open(os.path.join(ROOT, "tests", "golden", name)) as f:
            return json.load(f)
    return load


@pytest.fixture(scope="module")
def ctx():
    """A library context with a 4 GiB arena on cuda:0 (fp32 contractions)."""
    if not gpu_available():
        pytest.skip("no GPU")
    import transformer_fwd_bwd_amd as T
    c = T.Context(arena_bytes=4 << 30, precision="fp32")
    yield c
    c.close()
