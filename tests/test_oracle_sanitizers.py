"""The fp64 oracle under gcc's AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c includes the oracle's C source and calls every
entry point over seeded random shapes and edge cases with exactly sized
buffers; this test builds it with both sanitizers (any report is fatal) and
runs it on the CPU.  It checks memory safety and defined behaviour only; the
oracle's results are pinned by the other CPU tests.
"""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
MAIN = os.path.join(HERE, "oracle_sanitize_main.c")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc is not installed")
def test_oracle_is_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-ffp-contract=off", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", MAIN, "-lm", "-o", exe]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               OMP_NUM_THREADS="4")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report[-4000:]
    assert "runtime error" not in report and "AddressSanitizer" not in report, report[-4000:]
    assert "0 failed calls" in run.stdout
