"""Memory-wait placement in the compiled kernels (gfx950 assembly, built here
on the host; no GPU).

On gfx950 the vector memory counter counts stores as well as loads, so an
`s_waitcnt vmcnt` placed after a store waits for that store to complete.
Two placements cost measurable time and are guarded here:
  * the norm kernel at one chunk per lane (every instantiation with one
    segment) waits for its row's loads right after issuing them, and no
    vmcnt wait follows its first store (the compiler's own wait, placed
    after the residual store, made each wavefront wait for that store);
  * the standalone per-token quantiser issues every chunk's load before its
    first wait (loads under lane masks were waited for one at a time).
"""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "activation_fp8_quant_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"

pytestmark = pytest.mark.skipif(not os.path.exists(HIPCC) or shutil.which("bash") is None,
                                reason="needs hipcc")


def _asm(tmp_path, name):
    out = str(tmp_path / f"{name}.s")
    r = subprocess.run([HIPCC, "-x", "hip", "--offload-arch=gfx950", "--offload-device-only", "-S",
                        "-O3", "-std=c++17", f"-I{ROOT}/include", f"-I{CSRC}",
                        "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
                        os.path.join(CSRC, f"{name}.hip"), "-o", out],
                       capture_output=True, text=True, timeout=600)
    assert r.returncode == 0, r.stderr[-2000:]
    with open(out) as fh:
        return fh.read()


def _kernels(asm, prefix):
    """(mangled name, [memory events]) per kernel whose name starts with prefix:
    L = vector load, S = vector store, W = vmcnt wait, in program order."""
    out = []
    for m in re.finditer(r"^(" + prefix + r"\w*):[^\n]*\n(.*?)^\.Lfunc_end", asm, re.S | re.M):
        ev = []
        for line in m.group(2).splitlines():
            s = line.strip()
            if s.startswith(("global_load", "buffer_load")):
                ev.append("L")
            elif s.startswith(("global_store", "buffer_store")):
                ev.append("S")
            elif s.startswith("s_waitcnt") and "vmcnt" in s:
                ev.append("W")
        out.append((m.group(1), ev))
    return out


def test_norm_one_chunk_no_wait_after_store(tmp_path):
    # template arguments: dtype, mode, Gemma, chunks per lane, segments, aligned, fp32-direct
    ks = [(n, ev) for n, ev in _kernels(_asm(tmp_path, "afq_norm"), "_ZN3afq17norm_quant_kernel")
          if re.search(r"ILi\dELi\dELb\dELi1ELi1E", n)]
    assert len(ks) == 24, len(ks)  # 2 dtypes x 4 modes x 2 kinds x (1 or 2 quant inputs)
    for n, ev in ks:
        assert "S" in ev, n
        first_store = ev.index("S")
        assert "W" not in ev[first_store:], (n, "".join(ev))
        assert ev.index("W") > max(i for i, e in enumerate(ev) if e == "L" and i < first_store), n


def test_per_token_quant_loads_before_first_wait(tmp_path):
    ks = _kernels(_asm(tmp_path, "afq_quant"), "_ZN3afq16quant_row_kernel")
    assert len(ks) == 12, len(ks)  # 3 input dtypes x 1..4 chunks per lane
    for n, ev in ks:
        first_wait = ev.index("W")
        assert "L" not in ev[first_wait:], (n, "".join(ev))
