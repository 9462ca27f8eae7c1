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


def pytest_terminal_summary(terminalreporter):
    """Worst parity errors per workload (GPU runs only)."""
    try:
        import gpu_util
    except Exception:
        return
    if not gpu_util.WORST:
        return
    tr = terminalreporter
    tr.write_line("worst errors against the fp64 oracle, per workload "
                  "(bar: abs <= 5e-5 or rel <= 1e-3 per element):")
    for label in sorted(gpu_util.WORST):
        a, r, n = gpu_util.WORST[label]
        tr.write_line(f"  {label:<40s} max abs {a:.3e}  max rel {r:.3e}  "
                      f"({n} values)")
    path = os.environ.get("SPLITKV_PARITY_LOG")
    if path:
        import json
        with open(path, "w") as f:
            json.dump({k: {"max_abs": v[0], "max_rel": v[1], "values": v[2]}
                       for k, v in sorted(gpu_util.WORST.items())}, f,
                      indent=1)
