"""The step scheduler's host code under the address and undefined-behaviour
sanitizers (CPU only): tests/sched_fuzz.cpp drives random configurations and
random submit/step interleavings through mab_sched_* built with g++."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(shutil.which("g++") is None, reason="g++ not installed")
def test_scheduler_under_sanitizers(tmp_path):
    exe = tmp_path / "sched_fuzz"
    cmd = ["g++", "-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "sched_fuzz.cpp"),
           os.path.join(ROOT, "mixed_attention_block_amd", "csrc", "sched.cpp"), "-o", str(exe)]
    subprocess.run(cmd, check=True, capture_output=True, text=True)
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=1:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe), "300"], capture_output=True, text=True, env=env, timeout=300)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok 300")
