"""The host dual (csrc/planner.cpp, pure host C++) built with AddressSanitizer
and UndefinedBehaviorSanitizer by the host compiler and run on seeded random
tables by tests/native/planner_sanitize.cpp, which also checks each result
against the dual's contract (choices in range, bytes within the budget, every
choice minimal in D + lambda * bytes at the returned lambda, minimum-byte
choices when the budget is infeasible).  Host code only: no GPU code is built
with a sanitizer."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "kv_cache_compression_jolt_amd", "csrc")


@pytest.mark.timeout(300)
def test_planner_under_asan_ubsan(tmp_path):
    gxx = shutil.which("g++")
    if gxx is None:
        pytest.skip("no host C++ compiler")
    exe = str(tmp_path / "planner_sanitize")
    cmd = [gxx, "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-ffp-contract=off", "-I" + os.path.join(ROOT, "include"), "-I" + CSRC,
           os.path.join(CSRC, "planner.cpp"), os.path.join(ROOT, "tests", "native", "planner_sanitize.cpp"),
           "-pthread", "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:verify_asan_link_order=0", UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=240)
    assert r.returncode == 0, (r.stdout[-2000:], r.stderr[-4000:])
    assert "planner sanitize: 0 failures" in r.stdout
