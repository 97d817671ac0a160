"""Build libfa.so (the gfx950 HIP kernels and their C-ABI) in-tree with hipcc."""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
SRC = os.path.join(PKG, "csrc", "fa_abi.hip")
OUT = os.path.join(PKG, "libfa.so")
# the check build: every workgroup barrier waits for all outstanding memory operations
# first; tests compare its outputs with libfa.so's bit for bit
DEBUG_OUT = os.path.join(PKG, "libfa_debug.so")
DEBUG_FLAGS = ("-DFA_DEBUG_FULL_BARRIER",)

HIPCC_FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    "-Wall",
    # keep the compiler from emitting packed-fp32 VALU instructions
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
]


def build(out: str = OUT, extra=()) -> str:
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = out + ".tmp"
    cmd = [hipcc, *HIPCC_FLAGS, *extra, "-I", os.path.join(ROOT, "include"), "-o", tmp, SRC]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)  # atomic: a reader never sees a half-written library
    return out


def build_all() -> None:
    """Both libraries, compiled in parallel."""
    import concurrent.futures as cf
    with cf.ThreadPoolExecutor(2) as ex:
        for f in [ex.submit(build), ex.submit(build, DEBUG_OUT, DEBUG_FLAGS)]:
            f.result()


if __name__ == "__main__":
    if sys.argv[1:2] == ["--all"]:
        build_all()
    else:
        print(build(*(sys.argv[1:2] or [])))
