"""Build libsplitkv.so (gfx950) in-tree with hipcc.

    python -m decode_attention_gqa_amd.build        # or build() from Python

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


def _compile(src: str) -> tuple[str, str]:
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *CFLAGS, "-Rpass-analysis=kernel-resource-usage", "-c",
           os.path.join(CSRC, src), "-o", obj]
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


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
