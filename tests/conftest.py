import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU; runs the HIP path")


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def ctx():
    """One library context for the GPU tests of a session."""
    from tests.gpu_helpers import require_gpu
    require_gpu()
    import dense_linear_projection_amd as dlp
    h = dlp.proj_create(0)
    yield h
    dlp.proj_destroy(h)
