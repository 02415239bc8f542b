"""Host code under AddressSanitizer and UndefinedBehaviorSanitizer (CPU).

Three standalone programs are built with g++/gcc and the sanitizers, with no
HIP code in them:
  * abi_fuzz: the C ABI's validation (afq_abi.cpp) against stub launchers
    that check the invariants the kernels rely on, over 200,000 random
    descriptors (valid and invalid sizes, strides, pointers, enums);
  * oracle_run: every path of the CPU oracle on random and edge-case rows;
  * shape_check: the launch-shape rules (afq_shape.hpp) over every row width
    and a spread of row counts and compute-unit counts, against what the
    kernels assume of a shape, the rule's measured picks, and the flat
    kernels' division by the chunks per row against exact division.
Any sanitizer report, violated invariant or undocumented status fails.
"""
import os
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HERE = os.path.join(ROOT, "tests", "host_sanitize")
SAN = ["-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=all",
       "-fno-omit-frame-pointer"]

pytestmark = pytest.mark.skipif(shutil.which("g++") is None or shutil.which("gcc") is None,
                                reason="needs the host compilers")


def _run(cmd, **kw):
    return subprocess.run(cmd, capture_output=True, text=True, timeout=300, **kw)


def test_abi_validation_fuzz(tmp_path):
    exe = str(tmp_path / "abi_fuzz")
    b = _run(["g++", "-std=c++17", *SAN, f"-I{ROOT}/include",
              f"-I{ROOT}/activation_fp8_quant_amd/csrc",
              f"{ROOT}/activation_fp8_quant_amd/csrc/afq_abi.cpp", f"{HERE}/abi_fuzz.cpp", "-o", exe])
    assert b.returncode == 0, b.stderr
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=0"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert r.stdout.count(" 0:") == 4, r.stdout


def test_oracle_paths(tmp_path):
    exe = str(tmp_path / "oracle_run")
    b = _run(["gcc", "-std=c11", *SAN, f"{ROOT}/oracle/afq_oracle.c", f"{HERE}/oracle_run.c",
              "-o", exe, "-lm", "-lpthread"])
    assert b.returncode == 0, b.stderr
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "oracle paths ok" in r.stdout


def test_launch_shapes(tmp_path):
    exe = str(tmp_path / "shape_check")
    b = _run(["g++", "-std=c++17", *SAN, f"-I{ROOT}/activation_fp8_quant_amd/csrc",
              f"{HERE}/shape_check.cpp", "-o", exe])
    assert b.returncode == 0, b.stderr
    r = _run([exe], env=dict(os.environ, ASAN_OPTIONS="detect_leaks=1"))
    assert r.returncode == 0, r.stdout + r.stderr
    assert "runtime error" not in r.stderr and "ERROR: AddressSanitizer" not in r.stderr
    assert "launch shapes ok" in r.stdout
