import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


# A host-side sanitizer build of the library to load instead of the product
# one (set by tests/test_sanitizers.py for the child process it runs).
if os.environ.get("GDR_TEST_LIBRARY"):
    from chunkwise_gated_delta_cumsum_amd import binding as _binding
    _binding.LIB_PATH = os.environ["GDR_TEST_LIBRARY"]


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


@pytest.fixture(scope="session")
def gpu_lib():
    """The product binding, built HIP library loaded; skips without a GPU."""
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import chunkwise_gated_delta_cumsum_amd as gdr
    gdr.load()                       # raises if the HIP library is missing
    return gdr
