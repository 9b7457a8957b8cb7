"""The library's host-side argument checks and launch plan, compiled on their
own with g++ under the address and undefined-behaviour sanitizers (no HIP
runtime, no GPU) and driven through every precondition of the C ABI
(tests/host_check.cpp): each returns its MONO_E* code with a message, and
the workspace layouts and launch plans keep the invariants the kernels rely
on, the chunk-local instance being refused whenever its chunk items would
not all be resident at once."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "sparse_paged_decode_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not available")
def test_host_checks_under_sanitizers(tmp_path):
    exe = tmp_path / "host_check"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-fno-omit-frame-pointer", "-Wall", "-Werror", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_check.cpp"), os.path.join(CSRC, "plan.cpp"), "-o", str(exe)]
    build = subprocess.run(cmd, capture_output=True, text=True)
    assert build.returncode == 0, build.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="abort_on_error=0:halt_on_error=1", UBSAN_OPTIONS="halt_on_error=1")
    run = subprocess.run([str(exe)], capture_output=True, text=True, env=env, timeout=300)
    assert run.returncode == 0, (run.stdout + run.stderr)[-4000:]
    assert ", 0 failed" in run.stdout
