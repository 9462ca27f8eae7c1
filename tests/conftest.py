import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)
TESTS = os.path.dirname(os.path.abspath(__file__))
if TESTS not in sys.path:
    sys.path.insert(0, TESTS)


def pytest_configure(config):
    config.addinivalue_line(
        "markers", "gpu: needs an MI355X (gfx950) GPU and the built HIP library")


def _ensure_library():
    """Build libsplitkv.so only when nothing is built yet."""
    lib = os.path.join(ROOT, "decode_attention_gqa_amd", "libsplitkv.so")
    if not os.path.exists(lib):
        from decode_attention_gqa_amd import build
        build.build()
    return lib


import pytest  # noqa: E402


@pytest.fixture(scope="session")
def splitkv_lib_path():
    return _ensure_library()
