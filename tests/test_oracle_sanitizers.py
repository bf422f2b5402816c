"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and driven through every C entry point on tiny ragged inputs
(tests/oracle_sanitize_driver.c): no out-of-bounds access, leak, use after free
or undefined behaviour on the paths the parity tests rely on.  The build is
serial (no OpenMP) so that the report is deterministic."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE_C = os.path.join(ROOT, "oracle", "mla_oracle.c")
DRIVER_C = os.path.join(ROOT, "tests", "oracle_sanitize_driver.c")


def test_oracle_under_asan_and_ubsan(tmp_path):
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not available")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = [gcc, "-std=c11", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", ORACLE_C, DRIVER_C, "-o", exe, "-lm"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0 and "asan" in r.stderr.lower() and "cannot find" in r.stderr.lower():
        pytest.skip("sanitizer runtime not installed")
    assert r.returncode == 0, r.stderr
    # (the runtime need not come first among the process's libraries: the
    # environment may preload others)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "ERROR: AddressSanitizer" not in run.stderr and "runtime error" not in run.stderr, run.stderr
    assert "invalid items" in run.stdout
