"""The library's host-only code under AddressSanitizer and
UndefinedBehaviorSanitizer, on the CPU: config checks, the parameter and
arena layouts (with and without debug guard regions) and the matmul split
plans they size, the 16-bit widening, checkpoint headers and the token-file
loader, well-formed and malformed (tests/host_sanitize_driver.cpp).  The
sources are the library's own (host.cpp, plan.cpp, loader.cpp) built with
g++; any finding aborts the run (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "transformer_lm_step_train_amd", "csrc")


@pytest.mark.skipif(shutil.which("g++") is None, reason="needs g++")
def test_host_code_under_sanitizers(tmp_path):
    exe = os.path.join(tmp_path, "host_driver")
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wextra", "-Wno-unused-parameter",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC,
           os.path.join(ROOT, "tests", "host_sanitize_driver.cpp"),
           os.path.join(CSRC, "host.cpp"), os.path.join(CSRC, "plan.cpp"),
           os.path.join(CSRC, "loader.cpp"), "-o", exe]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-4000:]
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    data = os.path.join(tmp_path, "files")
    os.makedirs(data)
    r = subprocess.run([exe, data], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-4000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr
