"""Host check of the kernels' workgroup order (work_item in csrc/fa_common.hpp, a
host-and-device function): tests/work_item_check.cpp is compiled with hipcc for the
host and run; it checks that every grid shape maps its workgroups onto the (head,
tile) items one to one, with and without the causal weight-sorted list, and that the
sorted list reaches each XCD heaviest first.  No GPU is needed."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(HERE, "..", "flashattention_tiling_online_amd", "csrc")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
def test_work_item_is_a_bijection_and_heaviest_first(tmp_path):
    exe = tmp_path / "work_item_check"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC, "-o", str(exe),
           os.path.join(HERE, "work_item_check.cpp")]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-2000:]
    run = subprocess.run([str(exe)], capture_output=True, text=True, timeout=120)
    assert run.returncode == 0 and run.stdout.startswith("ok"), run.stdout + run.stderr
