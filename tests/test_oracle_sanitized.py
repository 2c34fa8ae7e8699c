"""The oracle built with AddressSanitizer and UndefinedBehaviorSanitizer (gcc,
host code only) and run through every entry point on small edge-case inputs
by tests/oracle_sanitize_driver.c: out-of-bounds indexing, use after free,
leaks and undefined arithmetic in the oracle fail this test."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
def test_oracle_under_sanitizers(tmp_path):
    exe = tmp_path / "oracle_asan"
    cmd = ["gcc", "-O1", "-g", "-std=c99", "-fno-omit-frame-pointer", "-ffp-contract=off",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
           os.path.join(ROOT, "oracle", "oracle.c"), os.path.join(HERE, "oracle_sanitize_driver.c"),
           "-o", str(exe), "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True)
    if build.returncode != 0 and "sanitize" in build.stderr:
        pytest.skip("this gcc has no sanitizer runtime: " + build.stderr.strip().splitlines()[-1])
    assert build.returncode == 0, build.stderr
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=120)
    assert run.returncode == 0, run.stdout + run.stderr
    assert "runtime error" not in run.stderr, run.stderr
    assert "ERROR: AddressSanitizer" not in run.stderr, run.stderr
    assert run.stdout.strip().endswith("rc 0"), run.stdout
