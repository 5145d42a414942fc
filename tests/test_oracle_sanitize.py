"""The CPU oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(g++, host code only) and driven through every entry point on small random
inputs (tests/oracle_sanitize_driver.cpp): no sanitizer report."""
import os
import shutil
import subprocess
import tempfile

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_oracle_under_asan_and_ubsan():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitize")
        subprocess.check_call(["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
                               "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
                               os.path.join(HERE, "oracle_sanitize_driver.cpp"), "-o", exe])
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "oracle sanitize run ok" in r.stdout
        assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr, r.stderr
