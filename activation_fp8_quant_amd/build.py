"""Build libafq.so (HIP kernels for gfx950 + the C ABI) in-tree with hipcc.

    python -m activation_fp8_quant_amd.build

The library is placed next to this file so that it travels with the source
tree.  Always recompiles (a build check must compile).
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
INCLUDE = os.path.join(ROOT, "include")
BUILD = os.path.join(HERE, "_build")
LIB = os.path.join(HERE, "libafq.so")

HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
ARCH = "gfx950"

# Packed fp32 VALU forms are kept out of the generated code.
NO_PACKED_FP32 = ["-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]
COMMON = ["-O3", "-std=c++17", "-fPIC", "-Wall", f"-I{INCLUDE}", f"-I{CSRC}"]


def _run(cmd):
    print("+", " ".join(cmd), flush=True)
    subprocess.check_call(cmd)


def _silu_table() -> None:
    """Generate the exact bf16(silu) table the 1x128 SiLU kernel reads for
    gates near a rounding midpoint (when missing or older than its
    generator)."""
    gen = os.path.join(CSRC, "gen_silu_table.py")
    inc = os.path.join(CSRC, "silu_bf16_table.inc")
    if not os.path.exists(inc) or os.path.getmtime(inc) < os.path.getmtime(gen):
        _run([sys.executable, gen, inc])


# one translation unit per kernel family
KERNEL_SOURCES = ("afq_norm.hip", "afq_act.hip", "afq_quant.hip")


def build(verbose: bool = True) -> str:
    os.makedirs(BUILD, exist_ok=True)
    _silu_table()
    cmds, objs = [], []
    for src in KERNEL_SOURCES:
        obj = os.path.join(BUILD, src.replace(".hip", ".o"))
        cmds.append([HIPCC, "-c", f"--offload-arch={ARCH}", *COMMON, *NO_PACKED_FP32,
                     "-x", "hip", os.path.join(CSRC, src), "-o", obj])
        objs.append(obj)
    # the ABI translation unit is plain host C++ (no HIP headers)
    aobj = os.path.join(BUILD, "afq_abi.o")
    cmds.append(["g++", "-c", "-O2", "-std=c++17", "-fPIC", "-Wall", "-Wextra",
                 f"-I{INCLUDE}", f"-I{CSRC}", os.path.join(CSRC, "afq_abi.cpp"), "-o", aobj])
    objs.append(aobj)
    procs = []
    for c in cmds:
        print("+", " ".join(c), flush=True)
        procs.append(subprocess.Popen(c))
    bad = [c for c, p in zip(cmds, procs) if p.wait() != 0]
    if bad:
        raise subprocess.CalledProcessError(1, bad[0])
    tmp = LIB + ".tmp"
    _run([HIPCC, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    build()
    sys.exit(0)
