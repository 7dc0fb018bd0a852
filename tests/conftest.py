import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")


@pytest.fixture(scope="session")
def O():
    import oracle
    return oracle.default()


@pytest.fixture(scope="session")
def K():
    """The product library; built in-tree first if nothing is built yet."""
    lib = os.path.join(ROOT, "quantized_decode_attention_amd", "libkvq.so")
    if not os.path.exists(lib):
        import importlib.util
        path = os.path.join(ROOT, "quantized_decode_attention_amd", "_build.py")
        spec = importlib.util.spec_from_file_location("kvq_build", path)
        _build = importlib.util.module_from_spec(spec)
        spec.loader.exec_module(_build)
        _build.build()
    import quantized_decode_attention_amd as K
    return K
