import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")

import pytest  # noqa: E402

LIB = os.path.join(ROOT, "hierarchical_sparse_attention_mean_amd", "liblighthouse.so")


@pytest.fixture(scope="session")
def lh():
    """The ctypes binding; builds the library first only if it is not built."""
    if not os.path.exists(LIB):
        from hierarchical_sparse_attention_mean_amd import build
        build.build()
    from hierarchical_sparse_attention_mean_amd import lighthouse
    return lighthouse
