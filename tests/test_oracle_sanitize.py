"""The oracle's C code under AddressSanitizer and UndefinedBehaviorSanitizer.

tests/oracle_sanitize_main.c calls every entry point of oracle/*.c on small
ragged shapes, row/key subsets, several thread counts and special values; it
is linked with the oracle sources into one executable built with
-fsanitize=address,undefined (no preloading: the executable carries the
sanitizer runtimes) and run in a subprocess.  Any report fails the test.
CPU only.
"""
import glob
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_under_asan_and_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    sources = sorted(glob.glob(os.path.join(ROOT, "oracle", "*.c")))
    assert sources, "no oracle sources"
    build = subprocess.run(
        ["gcc", "-O1", "-g", "-std=c11", "-pthread", "-fno-omit-frame-pointer",
         "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
         "-o", exe, os.path.join(ROOT, "tests", "oracle_sanitize_main.c"), *sources, "-lm"],
        capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    run = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=600)
    assert run.returncode == 0, (run.stdout + run.stderr)[-6000:]
    assert "ok" in run.stdout
    assert "runtime error" not in run.stderr and "AddressSanitizer" not in run.stderr, run.stderr[-6000:]
