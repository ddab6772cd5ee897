"""The oracle under AddressSanitizer and UndefinedBehaviorSanitizer: the
standalone driver (oracle/sanitize_driver.c) runs forward, backward and AdamW
on small ragged models (with and without rotary embedding), generation and
the loss-scale schedule, built as fp32 and as fp64.  Any finding aborts the
run (-fno-sanitize-recover=all)."""
import os
import shutil
import subprocess

import pytest

ORACLE = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "oracle")


@pytest.mark.skipif(shutil.which("gcc") is None, reason="needs gcc")
@pytest.mark.parametrize("fp64", [False, True])
def test_oracle_under_sanitizers(tmp_path, fp64):
    exe = os.path.join(tmp_path, "driver")
    cmd = ["gcc", "-std=gnu99", "-O1", "-g", "-fno-omit-frame-pointer",
           "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-Wall", "-Wno-unknown-pragmas", "-Wno-unused-function"]
    if fp64:
        cmd.append("-DORACLE_FP64")
    cmd += ["-I", ORACLE, os.path.join(ORACLE, "sanitize_driver.c"), "-o", exe, "-lm"]
    subprocess.run(cmd, check=True, capture_output=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0",
               UBSAN_OPTIONS="print_stacktrace=1")
    r = subprocess.run([exe], capture_output=True, text=True, env=env, timeout=300)
    assert r.returncode == 0, r.stdout[-2000:] + r.stderr[-4000:]
    assert r.stdout.strip().endswith("ok")
    assert "runtime error" not in r.stderr
