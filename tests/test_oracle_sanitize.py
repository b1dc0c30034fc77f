"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Compiles oracle/snack_oracle.c with gcc together with a driver that calls every
oracle entry point on small and degenerate inputs, and runs it: any
out-of-bounds access, leak, misaligned access, signed overflow or shift past
the width ends the run with a report and a non-zero status.
"""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not available")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(ROOT, "oracle", "snack_oracle.c"),
           os.path.join(ROOT, "tests", "oracle_sanitize_driver.c"), "-lm", "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    # verify_asan_link_order=0: a library preloaded into every process may come before the ASan runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert r.returncode == 0, f"sanitized oracle run failed ({r.returncode}):\n{r.stdout}\n{r.stderr[-4000:]}"
    assert "all cases ran" in r.stdout
