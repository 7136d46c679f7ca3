"""The C oracle under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c calls every entry point of oracle/csrc/oracle.c
on small edge-case layers with exactly sized buffers; built here with gcc's
-fsanitize=address,undefined (no recovery), any out-of-bounds access, use
after free or undefined operation in the oracle ends the run with a report.
The product library is HIP code for the GPU and is not built this way.
"""
import os
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "csrc", "oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_sanitize_main.c")


def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-fopenmp", "-ffp-contract=off", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", "-o", exe, ORACLE_C, DRIVER_C, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "asan" in build.stderr.lower():
        pytest.skip("gcc has no sanitizer runtime here:\n" + build.stderr)
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, OMP_NUM_THREADS="2",
               ASAN_OPTIONS="detect_leaks=0:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    report = run.stdout + run.stderr
    assert run.returncode == 0, report
    assert "runtime error" not in report and "ERROR: AddressSanitizer" not in report, report
    assert "all calls clean" in run.stdout
