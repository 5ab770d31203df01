import pytest
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
HERE = os.path.dirname(os.path.abspath(__file__))
if HERE not in sys.path:
    sys.path.insert(0, HERE)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture
def tile(request):
    """Force one GEMM kernel variant (a name of mixq.GEMM_VARIANTS) for the
    test, then restore the automatic choice."""
    from mixed_precision_quantized_amax_amd import mixq
    mixq.set_gemm_variant(request.param)
    yield request.param
    mixq.set_gemm_variant("auto")
