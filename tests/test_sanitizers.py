"""CPU: the host code under AddressSanitizer and UndefinedBehaviorSanitizer.

Builds libsplitkv.so (host code instrumented, device code as usual) and the C
oracle with both sanitizers (`python -m decode_attention_gqa_amd.build
--sanitize`), then runs the oracle pins, the mutation tests, the page
accounting and the C-ABI validation tests in a child process that preloads
the sanitizer runtime and loads the two instrumented builds. Any report
aborts the child, so the run must end clean. ("Red Lite dev35 — long-context
decode: grouped split-K attention", Validation, reports a sanitizer build
with no warnings.)
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHECKS = ["tests/test_oracle_pins.py", "tests/test_oracle_mutants.py",
          "tests/test_page_accounting.py", "tests/test_abi.py"]


def _has_gpu():
    try:
        import torch
        return torch.cuda.device_count() > 0
    except Exception:
        return False


@pytest.mark.skipif(_has_gpu(), reason="the ABI validation cases pass fake "
                    "pointers and run on GPU-less hosts only")
def test_cpu_checks_clean_under_asan_ubsan():
    sys.path.insert(0, ROOT)
    from decode_attention_gqa_amd import build
    san = build.build_sanitized()
    env = dict(os.environ)
    env.update(san)
    probe = subprocess.run(
        [sys.executable, "-c",
         "import oracle, decode_attention_gqa_amd as skv\n"
         "print(oracle.load()._name)\nprint(skv.load()._name)\n"
         "maps = open('/proc/self/maps').read()\n"
         "print('libclang_rt.asan' in maps)"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=600)
    assert probe.returncode == 0, probe.stderr[-3000:]
    lines = probe.stdout.split()
    assert lines[0] == san["SPLITKV_ORACLE_LIB"]
    assert lines[1] == san["SPLITKV_LIB"]
    assert lines[2] == "True"
    run = subprocess.run(
        [sys.executable, "-m", "pytest", *CHECKS, "-m", "not gpu", "-q",
         "-p", "no:cacheprovider"],
        cwd=ROOT, env=env, capture_output=True, text=True, timeout=1200)
    out = run.stdout + run.stderr
    assert run.returncode == 0, out[-4000:]
    assert "AddressSanitizer" not in out and "runtime error:" not in out
    assert " passed" in out
