"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer (host
code only): tests/oracle_sanitize_main.c drives every entry point of
oracle/pivot_oracle.c on small ragged shapes; the build aborts on the first
out-of-bounds access, leak or undefined operation."""
from __future__ import annotations

import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_clean_under_asan_and_ubsan(tmp_path):
    exe = tmp_path / "oracle_sanitized"
    cmd = ["gcc", "-O1", "-g", "-std=c11", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           os.path.join(HERE, "oracle_sanitize_main.c"), os.path.join(ROOT, "oracle", "pivot_oracle.c"),
           "-o", str(exe), "-lm"]
    subprocess.check_call(cmd)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=1", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    r = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "all checks passed" in r.stdout
