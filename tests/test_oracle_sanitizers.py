"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(gcc, host code only) and driven over small batches of every shape the
oracle handles (tests/oracle_sanitize_main.c): no out-of-bounds access, no
leak and no undefined behaviour may be reported."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_oracle_under_asan_and_ubsan(tmp_path):
    if shutil.which("gcc") is None:
        pytest.skip("gcc not found")
    exe = str(tmp_path / "oracle_sanitized")
    cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off", "-fno-fast-math",
           "-fno-omit-frame-pointer", "-fsanitize=address,undefined", "-static-libasan",
           "-fno-sanitize-recover=all", "-o", exe,
           os.path.join(ROOT, "oracle", "fpstok_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_main.c"), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:exitcode=42",
               UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
    assert "cases ok" in r.stdout
