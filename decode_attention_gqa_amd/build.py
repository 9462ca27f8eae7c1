"""Build libsplitkv.so (gfx950) in-tree with hipcc.

    python -m decode_attention_gqa_amd.build        # or build() from Python
    python -m decode_attention_gqa_amd.build --sanitize
        # host code under AddressSanitizer + UndefinedBehaviorSanitizer, and
        # the C oracle likewise, into _build/sanitize/ (CPU checks only: the
        # device code is built as usual, the sanitizers apply to host code)

Every HIP source is compiled for gfx950 only. Packed-FP32 instruction
selection is switched off for the device code (-packed-fp32-ops); the host
pass prints a harmless warning that it does not know the feature. The
compiler's per-kernel resource report (VGPRs, spills, scratch, LDS) is saved
next to the objects so tests can check that no kernel uses scratch memory.
"""
from __future__ import annotations

import concurrent.futures as cf
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(ROOT, "_build", "splitkv")
LIB = os.path.join(PKG, "libsplitkv.so")
RESOURCE_REPORT = os.path.join(BUILD, "resource_usage.txt")

SOURCES = ["splitkv_host.hip", "splitkv_partial.hip",
           "splitkv_partial_valu.hip", "splitkv_partial_mfma.hip",
           "splitkv_combine.hip", "splitkv_append.hip", "splitkv_probe.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"
CFLAGS = ["-O3", "-std=c++17", "-fPIC", f"--offload-arch={ARCH}",
          "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
          "-Wall", "-Wno-unused-function", f"-I{INCLUDE}", f"-I{CSRC}"]


# Host-side sanitizer flags: each -fsanitize goes to the host compilation only
# (-Xarch_host), never to the gfx950 code.
SAN_FLAGS = ["-Xarch_host", "-fsanitize=address", "-Xarch_host",
             "-fsanitize=undefined", "-Xarch_host", "-fno-sanitize-recover=all",
             "-Xarch_host", "-fno-omit-frame-pointer", "-Xarch_host", "-g"]
SAN_DIR = os.path.join(ROOT, "_build", "sanitize")
CLANG = os.environ.get("CLANG", "/opt/rocm/llvm/bin/clang")


def _compile(src: str, build_dir: str = BUILD,
             extra: tuple = ()) -> tuple[str, str]:
    obj = os.path.join(build_dir, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, *extra, "-Rpass-analysis=kernel-resource-usage",
           "-c", os.path.join(CSRC, src), "-o", obj]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{p.stderr}")
    return obj, p.stderr


def build(verbose: bool = False) -> str:
    """Compile every source and link the shared library; returns its path."""
    os.makedirs(BUILD, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(_compile, SOURCES))
    objs = [o for o, _ in results]
    with open(RESOURCE_REPORT, "w") as f:
        for src, (_, log) in zip(SOURCES, results):
            f.write(f"### {src}\n")
            f.write("\n".join(l for l in log.splitlines()
                              if "remark:" in l or "Function Name" in l))
            f.write("\n")
    tmp = LIB + ".tmp"
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", "-o", tmp, *objs]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"link failed:\n{p.stderr}")
    os.replace(tmp, LIB)
    if verbose:
        print(f"built {LIB}")
    return LIB


def asan_runtime() -> str:
    """Path of the shared AddressSanitizer runtime of the ROCm clang (to be
    preloaded into the Python process that loads the sanitizer builds)."""
    p = subprocess.run([CLANG, "-print-file-name=libclang_rt.asan-x86_64.so"],
                       capture_output=True, text=True, check=True)
    return p.stdout.strip()


def build_sanitized(verbose: bool = False) -> dict:
    """libsplitkv.so and the oracle with AddressSanitizer and
    UndefinedBehaviorSanitizer on their host code, into _build/sanitize/.
    Returns the paths and the environment that runs the CPU checks on them:
        SPLITKV_LIB, SPLITKV_ORACLE_LIB  the two builds
        LD_PRELOAD                       the sanitizer runtime (prepended)
        ASAN_OPTIONS, UBSAN_OPTIONS      abort on the first report; leak
                                         checks off (the interpreter and
                                         torch keep memory until exit)"""
    os.makedirs(SAN_DIR, exist_ok=True)
    with cf.ThreadPoolExecutor(max_workers=min(8, os.cpu_count() or 1)) as ex:
        results = list(ex.map(lambda f: _compile(f, SAN_DIR, tuple(SAN_FLAGS)),
                              SOURCES))
    lib = os.path.join(SAN_DIR, "libsplitkv.so")
    cmd = [HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host",
           "-fsanitize=undefined", "-shared-libasan", "-o", lib,
           *[o for o, _ in results]]
    p = subprocess.run(cmd, capture_output=True, text=True)
    if p.returncode != 0:
        raise RuntimeError(f"sanitizer link failed:\n{p.stderr}")
    sys.path.insert(0, ROOT)
    import oracle
    olib = oracle.build(os.path.join(SAN_DIR, "liboracle.so"),
                        ("-g", "-fno-omit-frame-pointer",
                         "-fsanitize=address,undefined",
                         "-fno-sanitize-recover=all", "-shared-libasan"),
                        cc=CLANG)
    rt = asan_runtime()
    pre = os.environ.get("LD_PRELOAD", "")
    env = {"SPLITKV_LIB": lib, "SPLITKV_ORACLE_LIB": olib,
           "LD_PRELOAD": rt + (":" + pre if pre else ""),
           "ASAN_OPTIONS": "detect_leaks=0:halt_on_error=1:abort_on_error=1",
           "UBSAN_OPTIONS": "halt_on_error=1:print_stacktrace=1"}
    if verbose:
        for k, v in env.items():
            print(f"{k}={v}")
    return env


if __name__ == "__main__":
    if "--sanitize" in sys.argv[1:]:
        build_sanitized(verbose=True)
    else:
        build(verbose=True)
    sys.exit(0)
