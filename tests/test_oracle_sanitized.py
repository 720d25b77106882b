"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc), driven through
every entry point by oracle/sanitize_check.c with buffers of exactly the sizes its layout rules
give: an out-of-bounds access or undefined behaviour ends the run with a report."""
import os
import shutil
import subprocess

import pytest

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_runs_clean_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "sanitize_check")
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-ffp-contract=off", "-o", exe, os.path.join(ORACLE, "oracle.c"), os.path.join(ORACLE, "sanitize_check.c"),
           "-lm"]
    b = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    if b.returncode != 0 and "asan" in b.stderr.lower():
        pytest.skip("the sanitizer runtimes are not installed: " + b.stderr[-200:])
    assert b.returncode == 0, b.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, timeout=300, env=env)
    assert r.returncode == 0, r.stderr[-4000:]
    assert "sanitize_check: clean" in r.stdout
