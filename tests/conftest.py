import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU and the built libpolar")
    # tests/test_host_asan.py runs the ABI tests again in a child process against a build
    # whose host code carries AddressSanitizer; that child names the library here.
    alt = os.environ.get("POLAR_TEST_LIBRARY")
    if alt:
        from long_context_lm_amd import _lib
        print(f"[abi] library {_lib.load(alt)._name}", flush=True)


@pytest.fixture(scope="session")
def gpu_lib():
    """The loaded libpolar (GPU tests only); fails loudly when it is missing."""
    import torch
    if not torch.cuda.is_available():
        pytest.fail("GPU test collected but no GPU is visible")
    from long_context_lm_amd import _lib
    return _lib.load()
