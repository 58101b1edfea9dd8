"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc) and run
on every entry point with small and edge-case inputs (tests/sanitize/oracle_main.c): no
out-of-bounds access, leak, or undefined behaviour may be reported."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_asan_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fopenmp", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", os.path.join(ROOT, "oracle", "rtl_oracle.c"),
           os.path.join(ROOT, "tests", "sanitize", "oracle_main.c"), "-o", str(exe), "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, OMP_NUM_THREADS="2", ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0 and r.stdout.strip() == "OK", (r.returncode, r.stdout[-2000:], r.stderr[-4000:])
