"""Builds libmab.so in-tree for gfx950 with hipcc.

Usage: ``python -m mixed_attention_block_amd.build``.
"""

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
SRC = os.path.join(HERE, "csrc", "mab.hip")
SCHED = os.path.join(HERE, "csrc", "sched.cpp")  # host code: the step scheduler
PROBE = os.path.join(HERE, "csrc", "probe.hip")  # measurement probes (stream read, dense MFMA)
OUT = os.path.join(HERE, "libmab.so")

FLAGS = [
    "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared",
    # no packed fp32 arithmetic: its forms are avoided on this hardware
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # no operand holds a NaN (masked keys are -inf, unwritten bytes are zeroed
    # by their scale): max needs no NaN-quieting instructions
    "-fno-honor-nans",
    "-I" + os.path.join(ROOT, "include"),
    "-Wl,-rpath,/opt/rocm/lib",
]


def build(verbose=False):
    hipcc = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
    tmp = OUT + ".tmp"
    cmd = [hipcc] + FLAGS + [SRC, PROBE, SCHED, "-o", tmp]
    res = subprocess.run(cmd, capture_output=True, text=True)
    if res.returncode != 0:
        sys.stderr.write(res.stdout + res.stderr)
        raise RuntimeError("hipcc failed: " + " ".join(cmd))
    if verbose:
        noise = "packed-fp32-ops' is not a recognized feature"
        msg = "\n".join(l for l in (res.stdout + res.stderr).splitlines() if noise not in l)
        if msg.strip():
            sys.stderr.write(msg + "\n")
    os.replace(tmp, OUT)
    return OUT


if __name__ == "__main__":
    print(build(verbose=True))
