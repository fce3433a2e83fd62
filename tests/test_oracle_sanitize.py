"""Builds the CPU oracle (oracle/eqtp_oracle.c) together with a driver that
calls every one of its entry points (tests/oracle_sanitize_main.c) under
AddressSanitizer and UndefinedBehaviorSanitizer, and runs it: an
out-of-bounds access, a use after free, a leak, a signed overflow or any other
undefined operation anywhere in the oracle fails the test.  The driver runs
the convolution and the linear once on one thread and once on three (OpenMP),
so the threaded loops are covered too.  Host only."""
import os
import shutil
import subprocess

import pytest

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)


@pytest.mark.skipif(shutil.which("gcc") is None, reason="gcc not found")
def test_oracle_clean_under_asan_ubsan(tmp_path):
    exe = str(tmp_path / "oracle_sanitize")
    cmd = ["gcc", "-std=gnu11", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all", "-fopenmp",
           os.path.join(ROOT, "oracle", "eqtp_oracle.c"), os.path.join(HERE, "oracle_sanitize_main.c"),
           "-o", exe, "-lm"]
    build = subprocess.run(cmd, capture_output=True, text=True, timeout=300)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ)
    env["ASAN_OPTIONS"] = "detect_leaks=1:abort_on_error=0:halt_on_error=1"
    env["UBSAN_OPTIONS"] = "print_stacktrace=1:halt_on_error=1"
    # the sanitizer runtime has to be the first library loaded
    env.pop("LD_PRELOAD", None)
    run = subprocess.run([exe], capture_output=True, text=True, timeout=600, env=env)
    log = run.stdout + run.stderr
    assert run.returncode == 0, log[-6000:]
    assert "AddressSanitizer" not in log and "runtime error" not in log, log[-6000:]
    assert "all entry points clean" in run.stdout
