"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU only).

Two drivers under tests/sanitize/ are built with the sanitizers and run; each halts
on the first finding and prints "ok" when every call returned what it should:

* oracle_main.c links oracle/fa_oracle.c (gcc, -fsanitize=address,undefined, leak
  checking on) and calls every function the oracle exports on small inputs of each
  storage type, masks with a row that sees no key, dropout, gradients, and arguments
  the oracle must refuse;
* abi_main.cpp links the C-ABI (csrc/fa_abi.hip, hipcc with the sanitizers on the host
  side only; the device code is compiled but never run) and calls every entry point
  with arguments that its checks refuse before any HIP call: null, misaligned and
  out-of-range arguments, unknown enum values, sizes whose byte counts would wrap
  int64, masks and workspaces that do not fit.

No GPU is touched: the ABI driver makes no HIP call that reaches a device.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SAN = os.path.join(ROOT, "tests", "sanitize")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
HOST_SAN = ["-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
            "-Xarch_host", "-fno-sanitize-recover=all"]


def _run(exe, leaks):
    env = dict(os.environ, ASAN_OPTIONS=f"detect_leaks={int(leaks)}:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=120, env=env)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-4000:]


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_san")
    subprocess.run(["gcc", "-std=c11", "-O1", "-g", "-fsanitize=address,undefined",
                    "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
                    os.path.join(SAN, "oracle_main.c"), os.path.join(ROOT, "oracle", "fa_oracle.c"),
                    "-lm", "-lpthread", "-o", exe], check=True)
    _run(exe, leaks=True)


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="needs hipcc")
def test_abi_host_checks_under_asan_ubsan(tmp_path):
    obj = str(tmp_path / "fa_abi.o")
    exe = str(tmp_path / "abi_san")
    inc = ["-I", os.path.join(ROOT, "include")]
    # device code at -O1 (the least that keeps the DMA's inline-assembly operands in
    # scalar registers): it is compiled for the link but never launched
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O1",
                    "-Xarch_device", "-g0", "-g", "-std=c++17", "-fPIC", *HOST_SAN,
                    "-fno-omit-frame-pointer", "-Xclang", "-target-feature", "-Xclang",
                    "-packed-fp32-ops", *inc, "-c",
                    os.path.join(ROOT, "flashattention_tiling_online_amd", "csrc", "fa_abi.hip"),
                    "-o", obj], check=True, capture_output=True, timeout=600)
    subprocess.run([HIPCC, "-O1", "-g", "-std=c++17", *HOST_SAN, "-fno-omit-frame-pointer",
                    *inc, "-x", "c++", os.path.join(SAN, "abi_main.cpp"), "-x", "none", obj,
                    "-o", exe], check=True, capture_output=True, timeout=300)
    _run(exe, leaks=True)
