"""The launch geometry and the workspace layout, checked on the CPU.

tests/layout_check.cpp includes the library's source and, over a sweep of
shapes with the extremes (batch up to the ready list's limit and one past it,
gamma 1..63, vocabularies from 1 to past the row counter's 16 bits), checks
that every workgroup of every launch decodes to work inside the problem with
the kernels' own decode functions, that every workspace array fits its
region, and that sizes and refusals follow the stated limits.  No kernel runs.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "layout_check.cpp")
HIPCC = shutil.which("hipcc") or "/opt/rocm/bin/hipcc"


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc is not installed")
def test_launch_geometry_and_workspace_layout(tmp_path):
    exe = str(tmp_path / "layout_check")
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-I", os.path.join(HERE, "..", "include"), SRC, "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert " 0 failed checks" in run.stdout, run.stdout
