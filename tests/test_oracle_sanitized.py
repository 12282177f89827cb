"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
CPU only) and driven over every entry point at small shapes by
oracle/sanitize_driver.c: no out-of-bounds access, no use of freed memory,
no undefined arithmetic (signed overflow, bad shifts, misaligned access), and
every call returns what its contract states."""
import os
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
ORACLE = os.path.join(ROOT, "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_address_and_ub_sanitizers():
    with tempfile.TemporaryDirectory() as tmp:
        exe = os.path.join(tmp, "oracle_sanitized")
        cmd = ["gcc", "-std=c11", "-O1", "-g", "-ffp-contract=off",
               "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fno-omit-frame-pointer",
               os.path.join(ORACLE, "gr_oracle.c"), os.path.join(ORACLE, "sanitize_driver.c"),
               "-o", exe, "-lm"]
        b = subprocess.run(cmd, capture_output=True, text=True)
        if b.returncode != 0 and "asan" in (b.stderr + b.stdout).lower():
            pytest.skip("gcc cannot link the sanitizer runtimes here: " + b.stderr[-300:])
        assert b.returncode == 0, b.stderr
        env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0:verify_asan_link_order=0",
                   UBSAN_OPTIONS="print_stacktrace=1:halt_on_error=1")
        r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
        assert r.returncode == 0, r.stdout + r.stderr
        assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
        assert "all calls ok" in r.stdout
