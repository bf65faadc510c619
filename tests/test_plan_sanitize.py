"""The host plan (argument checks, chunk policy, workspace layout) built for
the CPU with the address and undefined-behaviour sanitizers and run over the
overflow shapes of RL-Kernel PR #495's INT_MAX review (V = 2147482624, N V
beyond 2^31) and a sweep of shapes; any sanitizer report fails the run."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
SRC = os.path.join(ROOT, "tests", "native", "plan_check.cpp")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_plan_under_sanitizers(tmp_path):
    exe = str(tmp_path / "plan_check")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer", "-fsanitize=address,undefined",
           "-fno-sanitize-recover=all", "-Wall", SRC, "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    # verify_asan_link_order=0: the environment may preload a library ahead of the sanitizer runtime
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "AddressSanitizer" not in r.stderr, r.stderr
    assert "0 failures" in r.stdout
