"""The attention library's host planner under the address and
undefined-behaviour sanitizers (CPU only).  tests/planner_fuzz.cpp sends
random layouts and batches, well formed and malformed, through
attention_workspace_bytes, kv_append_quant and mixed_attention_fwd (layout
and batch checks, launch classification, workspace sizing, launch tables).
The host side of the library is built with the sanitizers; its device code
is compiled without optimisation and never runs: the driver makes the calls
that would launch kernels only when no device is visible, so those launches
fail with a status."""

import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not installed")
def test_planner_under_sanitizers(tmp_path):
    exe = tmp_path / "planner_fuzz"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O1", "-Xarch_device", "-O0", "-g", "-std=c++17",
           "-Xarch_host", "-fsanitize=address", "-Xarch_host", "-fsanitize=undefined",
           "-Xarch_host", "-fno-sanitize-recover=all",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I" + os.path.join(ROOT, "include"), os.path.join(ROOT, "tests", "planner_fuzz.cpp"),
           os.path.join(ROOT, "mixed_attention_block_amd", "csrc", "mab.hip"), "-o", str(exe)]
    res = subprocess.run(cmd, capture_output=True, text=True)
    assert res.returncode == 0, res.stdout + res.stderr
    # the HIP runtime is not built with the sanitizer: leak reports from it are not the planner's
    env = dict(os.environ, ASAN_OPTIONS="detect_leaks=0:abort_on_error=0", UBSAN_OPTIONS="print_stacktrace=1",
               HIP_VISIBLE_DEVICES="")
    env.pop("LD_PRELOAD", None)
    res = subprocess.run([str(exe), "400"], capture_output=True, text=True, env=env, timeout=600)
    assert res.returncode == 0, res.stdout + res.stderr
    assert res.stdout.startswith("ok 400"), res.stdout
