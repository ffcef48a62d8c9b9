"""The oracle built for the host with AddressSanitizer and UndefinedBehaviorSanitizer (gcc) and run
through every entry point on small inputs with its edge cases (tests/oracle_sanitize_driver.c):
no invalid memory access, leak or undefined behaviour, and the driver's own checks pass."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "mla_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"),
           "-o", str(exe), "-lpthread", "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
