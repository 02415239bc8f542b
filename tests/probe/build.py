"""Build the test-only probe library (tests/probe/libafq_probe.so) with
hipcc for gfx950.  It holds element-wise probe kernels over the library's
device primitives; only the tests load it.

    python -m tests.probe.build
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(os.path.dirname(HERE))
CSRC = os.path.join(ROOT, "activation_fp8_quant_amd", "csrc")
LIB = os.path.join(HERE, "libafq_probe.so")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")


def build() -> str:
    tmp = LIB + ".tmp"
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-shared", "-Wall",
           f"-I{CSRC}", "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-x", "hip", os.path.join(HERE, "afq_probe.hip"), "-o", tmp]
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
