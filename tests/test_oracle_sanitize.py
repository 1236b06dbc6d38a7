"""The CPU oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): tests/oracle_sanitize_driver.c compiles the oracle's source into one
binary with the sanitizers and drives every entry point, its edge cases and its
argument-error paths; any out-of-bounds access, leak, or undefined operation
aborts the run."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
DRIVER = os.path.join(HERE, "oracle_sanitize_driver.c")
FLAGS = ["-std=c11", "-O1", "-g", "-fopenmp", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all"]


def test_oracle_under_sanitizers(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc is not available")
    exe = str(tmp_path / "oracle_sanitize")
    subprocess.run(["gcc", *FLAGS, DRIVER, "-o", exe, "-lm"], check=True,
                   capture_output=True, text=True)
    env = dict(os.environ, OMP_NUM_THREADS="3",
               ASAN_OPTIONS="abort_on_error=1:detect_leaks=1",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, r.stdout + r.stderr
    assert r.stdout.strip() == "OK", r.stdout + r.stderr
