"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer
(host code only) and driven through every exported function on exactly
sized buffers by oracle/sanitize_driver.c: any out-of-bounds access, leak or
undefined behaviour fails the run."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_address_and_ub_sanitizers():
    with tempfile.TemporaryDirectory() as d:
        exe = os.path.join(d, "oracle_sanitized")
        cmd = ["gcc", "-O1", "-g", "-fno-omit-frame-pointer", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-pthread",
               "-o", exe, os.path.join(ORACLE, "oracle.c"),
               os.path.join(ORACLE, "sanitize_driver.c"), "-lm"]
        subprocess.run(cmd, check=True, capture_output=True, text=True)
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
        assert "sanitizer run clean" in r.stdout
