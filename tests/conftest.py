import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def flush_print(*args):
    """Name the case before a GPU step, flushed, so a crash still says which."""
    print(*args, flush=True)
    sys.stdout.flush()


@pytest.fixture(scope="session")
def gpu_lib():
    """The HIP attention library, loaded from the in-tree build. Fails loudly
    (never falls back) when the library or the GPU is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test run without a visible GPU")
    import online_softmax_amd as osa
    osa.load()  # raises if the shared library is absent
    return osa
