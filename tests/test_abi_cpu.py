"""The C ABI on the CPU: libafq.so loads, exports every function that
include/afq.h declares, the Python binding's descriptor layouts match the C
header, and every validation error is reported without touching a GPU
(rejected calls return before any HIP call)."""
import ctypes
import os
import re
import subprocess

import pytest

import activation_fp8_quant_amd as afq

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "afq.h")


def _declared_functions():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\*?\s*(\w+)\s*\([^;]*\)\s*;", src, re.M)))


def test_library_exports_every_declared_function():
    names = _declared_functions()
    assert {"fused_add_rmsnorm_quant", "silu_mul_quant", "swiglu_oai_quant", "fp8_quant",
            "afq_status_string", "afq_abi_version", "afq_last_hip_error"} <= set(names)
    out = subprocess.check_output(["nm", "-D", "--defined-only", afq.library_path], text=True)
    exported = {line.split()[-1] for line in out.splitlines() if " T " in line}
    missing = [n for n in names if n not in exported]
    assert not missing, missing
    lib = afq.load()
    for n in names:
        assert hasattr(lib, n)


def test_abi_version_and_status_strings():
    assert afq.abi_version() == 4
    for st in range(0, -9, -1):
        s = afq.status_string(st)
        assert s and s != "unknown status"
    assert afq.status_string(-100) == "unknown status"
    assert afq.load().afq_last_hip_error() == 0


def test_descriptor_layout_matches_header(tmp_path):
    """Compile a C probe against include/afq.h and compare sizes/offsets."""
    probe = tmp_path / "probe.c"
    fields = {
        "afq_qact": ["values", "scales", "normed"],
        "afq_norm_seg": ["x", "x_row_stride", "weight", "cols", "out"],
        "afq_norm_desc": ["M", "nseg", "kind", "dtype", "mode", "eps", "quant_input", "residual_in",
                          "residual_out", "seg"],
        "afq_act_desc": ["M", "I", "gate_up", "gate_up_row_stride", "mode", "quant_input", "out"],
        "afq_quant_desc": ["M", "cols", "x", "x_row_stride", "dtype", "mode", "out"],
        "afq_swiglu_desc": ["act", "alpha", "beta", "limit"],
    }
    lines = ['#include <stdio.h>', '#include <stddef.h>', '#include "afq.h"', "int main(void){"]
    for st, fs in fields.items():
        lines.append(f'printf("{st} size %zu\\n", sizeof({st}));')
        for f in fs:
            lines.append(f'printf("{st} {f} %zu\\n", offsetof({st}, {f}));')
    lines.append("return 0;}")
    probe.write_text("\n".join(lines))
    exe = tmp_path / "probe"
    subprocess.check_call(["gcc", "-std=c11", f"-I{ROOT}/include", str(probe), "-o", str(exe)])
    c = {}
    for line in subprocess.check_output([str(exe)], text=True).splitlines():
        parts = line.split()
        c[tuple(parts[:-1])] = int(parts[-1])
    py = {"afq_qact": afq._QAct, "afq_norm_seg": afq._NormSeg, "afq_norm_desc": afq._NormDesc,
          "afq_act_desc": afq._ActDesc, "afq_quant_desc": afq._QuantDesc,
          "afq_swiglu_desc": afq._SwigluDesc}
    for st, cls in py.items():
        assert c[(st, "size")] == ctypes.sizeof(cls), st
        for f in fields[st]:
            assert c[(st, f)] == getattr(cls, f).offset, (st, f)


# ------------------------------------------------------------- validation
A16 = 0x10000  # a fake, 16-byte aligned "device" address (never dereferenced)


def _norm(M=4, cols=256, mode=afq.MXFP8, **kw):
    d = afq._NormDesc()
    d.M, d.nseg, d.kind, d.dtype, d.mode, d.eps = M, 1, afq.GEMMA, 0, mode, 1e-6
    s = d.seg[0]
    s.x, s.x_row_stride, s.weight, s.cols = A16, cols, A16 * 2, cols
    s.out.values, s.out.scales, s.out.normed = A16 * 3, A16 * 4, None
    for k, v in kw.items():
        setattr(d, k, v)
    return d


def _call_norm(d):
    return afq.load().fused_add_rmsnorm_quant(ctypes.byref(d), None)


def test_norm_validation_errors():
    lib = afq.load()
    assert lib.fused_add_rmsnorm_quant(None, None) == -1
    assert _call_norm(_norm(M=-1)) == -2
    assert _call_norm(_norm(cols=48)) == -2                    # not a multiple of 32 (MX)
    assert _call_norm(_norm(cols=256 + 32, mode=afq.BLOCK128)) == -2
    assert _call_norm(_norm(cols=65536)) == -2                 # above AFQ_MAX_COLS
    assert _call_norm(_norm(nseg=3)) == -2
    assert _call_norm(_norm(mode=7)) == -7
    assert _call_norm(_norm(kind=5)) == -7
    assert _call_norm(_norm(dtype=2)) == -4                    # fp32 norm input
    assert _call_norm(_norm(eps=-1.0)) == -7
    assert _call_norm(_norm(eps=float("nan"))) == -7
    assert _call_norm(_norm(M=2 ** 31)) == -2                  # above AFQ_MAX_ROWS
    d = _norm()
    d.seg[0].x_row_stride = 2 ** 40 + 256                      # above AFQ_MAX_ROW_STRIDE
    assert _call_norm(d) == -2
    d = _norm(M=1 << 20)
    d.seg[0].out.values = (1 << 64) - (1 << 24)                # would run past the address space
    assert _call_norm(d) == -2
    assert _call_norm(_norm(quant_input=3)) == -7              # unknown quant_input
    assert _call_norm(_norm(quant_input=afq.QIN_FP32)) == -6   # fp32-direct: not with MXFP8
    assert _call_norm(_norm(quant_input=afq.QIN_BF16)) == -6   # bf16-first: SiLU only
    d = _norm()
    d.seg[0].x_row_stride = 128                                # stride < cols
    assert _call_norm(d) == -2
    d = _norm()
    d.seg[0].x = None
    assert _call_norm(d) == -1
    d = _norm()
    d.seg[0].x = A16 + 8                                       # misaligned
    assert _call_norm(d) == -3
    d = _norm()
    d.seg[0].out.scales = A16 * 4 + 2                          # scales need 4-byte alignment
    assert _call_norm(d) == -3
    d = _norm()
    d.residual_in = A16 * 8                                    # residual_in without residual_out
    assert _call_norm(d) == -1
    d = _norm(nseg=2)
    d.seg[1] = d.seg[0]
    d.residual_in, d.residual_out = A16 * 8, A16 * 9
    assert _call_norm(d) == -2                                 # residual with two segments
    d = _norm()
    d.seg[0].out.scales = A16 * 3 + 64                         # scales inside the codes
    assert _call_norm(d) == -5
    d = _norm()
    d.seg[0].out.values = A16                                  # codes over the input
    assert _call_norm(d) == -5
    d = _norm()
    d.residual_in, d.residual_out = A16 * 8, A16 * 8 + 16      # partial residual overlap
    assert _call_norm(d) == -5
    # M == 0: OK and nothing enqueued, even with NULL pointers
    d = _norm(M=0)
    d.seg[0].x = None
    assert _call_norm(d) == 0


def test_act_and_quant_validation_errors():
    lib = afq.load()
    d = afq._ActDesc()
    d.M, d.I, d.gate_up, d.gate_up_row_stride, d.mode = 4, 768, A16, 1536, afq.MXFP8
    d.out.values, d.out.scales = A16 * 64, A16 * 128
    assert lib.silu_mul_quant(None, None) == -1
    d.mode = afq.PER_TOKEN
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -6
    d.mode, d.quant_input = afq.MXFP8, 3
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -7     # unknown quant_input
    d.quant_input = afq.QIN_FP32
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -6     # fp32-direct: norm only
    d.mode, d.quant_input = afq.BLOCK128, afq.QIN_BF16
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -6     # bf16-first: MXFP8 only
    d.quant_input = afq.QIN_DEFAULT
    d.mode = afq.BLOCK128                                       # 768 % 128 == 0 but ...
    d.I = 96
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -2     # 96 % 128 != 0
    d.I, d.gate_up_row_stride = 768, 1000
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -2     # stride < 2I
    d.gate_up_row_stride = 1540
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -3     # pitch not 16-byte multiple
    d.gate_up_row_stride = 1536
    d.out.values = A16 + 32                                    # codes inside the input
    assert lib.silu_mul_quant(ctypes.byref(d), None) == -5
    q = afq._QuantDesc()
    q.M, q.cols, q.x, q.x_row_stride, q.dtype, q.mode = 2, 256, A16, 256, 2, afq.MXFP8
    q.out.values, q.out.scales = A16 * 64, A16 * 128
    q.out.normed = A16 * 256
    assert lib.fp8_quant(ctypes.byref(q), None) == -7          # no normed output here
    q.out.normed = None
    q.dtype = 9
    assert lib.fp8_quant(ctypes.byref(q), None) == -7
    q.dtype, q.cols = 2, 100
    assert lib.fp8_quant(ctypes.byref(q), None) == -2


def test_copy_only_validation():
    """values and scales both NULL: a copy-only launch (the first kernel of
    an unfused chain).  Its copy is required, its widths need only be whole
    chunks, it reads the default input only, and one of values / scales
    alone is a NULL error."""
    lib = afq.load()

    def copy_only(**kw):
        d = _norm(**kw)
        d.seg[0].out.values, d.seg[0].out.scales, d.seg[0].out.normed = None, None, A16 * 3
        return d

    assert _call_norm(copy_only(M=0, cols=48)) == 0             # width 48: no 1x32 groups needed
    assert _call_norm(copy_only(M=0, cols=44)) == -2            # still whole 8-element chunks
    assert _call_norm(copy_only(quant_input=afq.QIN_FP32, mode=afq.BLOCK128)) == -6
    d = copy_only()
    d.seg[0].out.normed = None                                  # nothing to write
    assert _call_norm(d) == -1
    d = copy_only()
    d.seg[0].out.scales = A16 * 4                               # scales without codes
    assert _call_norm(d) == -1
    d = copy_only()
    d.seg[0].out.normed = A16 * 3 + 8                           # misaligned copy
    assert _call_norm(d) == -3
    d = copy_only()
    d.seg[0].out.normed = A16                                   # copy over the input
    assert _call_norm(d) == -5
    d = copy_only(nseg=2)                                       # one segment quantised, one not
    d.seg[1] = d.seg[0]
    d.seg[1].x, d.seg[1].weight = A16 * 16, A16 * 17
    d.seg[1].out.values, d.seg[1].out.scales, d.seg[1].out.normed = A16 * 18, A16 * 19, A16 * 20
    assert _call_norm(d) == -1
    a = afq._ActDesc()
    a.M, a.I, a.gate_up, a.gate_up_row_stride, a.mode = 0, 200, A16, 400, afq.BLOCK128
    a.out.normed = A16 * 64
    assert lib.silu_mul_quant(ctypes.byref(a), None) == 0      # 200 % 128 != 0: fine without groups
    a.M = 4
    a.quant_input = afq.QIN_BF16
    a.mode = afq.MXFP8
    assert lib.silu_mul_quant(ctypes.byref(a), None) == -6     # bf16-first: a quantiser input
    a.quant_input = afq.QIN_DEFAULT
    a.out.normed = None
    assert lib.silu_mul_quant(ctypes.byref(a), None) == -1
    a.out.normed, a.out.values = A16 * 64, A16 * 128
    assert lib.silu_mul_quant(ctypes.byref(a), None) == -2     # quantising: 200 is no 1x32 width
    a.I, a.gate_up_row_stride = 256, 512
    assert lib.silu_mul_quant(ctypes.byref(a), None) == -1     # codes without scales
    a.out.values = None
    a.mode = afq.PER_TOKEN
    assert lib.silu_mul_quant(ctypes.byref(a), None) == -6     # no per-token activation


def test_swiglu_validation_errors():
    """The clamped SwiGLU entry: MXFP8 only; alpha and beta finite, limit
    positive (infinity allowed); the activation descriptor is checked as
    silu_mul_quant checks it."""
    lib = afq.load()
    inf, nan = float("inf"), float("nan")

    def desc(**kw):
        d = afq._SwigluDesc()
        a = d.act
        a.M, a.I, a.gate_up, a.gate_up_row_stride, a.mode = 0, 768, A16, 1536, afq.MXFP8
        a.out.values, a.out.scales = A16 * 64, A16 * 128
        d.alpha, d.beta, d.limit = 1.702, 1.0, 7.0
        for k, v in kw.items():
            setattr(d, k, v)
        return d

    def call(d):
        return lib.swiglu_oai_quant(ctypes.byref(d), None)

    assert lib.swiglu_oai_quant(None, None) == -1
    assert call(desc()) == 0                                   # M = 0: nothing enqueued
    assert call(desc(limit=inf)) == 0
    for bad in (dict(alpha=inf), dict(alpha=nan), dict(beta=-inf), dict(beta=nan),
                dict(limit=0.0), dict(limit=-1.0), dict(limit=nan), dict(limit=-inf)):
        assert call(desc(**bad)) == -7, bad
    d = desc()
    d.act.mode = afq.BLOCK128
    assert call(d) == -6
    d.act.mode = afq.PER_TOKEN
    assert call(d) == -6
    d.act.mode = 7
    assert call(d) == -7
    d = desc()
    d.act.quant_input = afq.QIN_FP32
    assert call(d) == -6
    d.act.quant_input = afq.QIN_BF16
    assert call(d) == 0
    d = desc()
    d.act.M, d.act.I = 4, 100
    assert call(d) == -2                                       # no 1x32 width
    d.act.I, d.act.gate_up_row_stride = 768, 1540
    assert call(d) == -3
    d.act.gate_up_row_stride = 1536
    d.act.out.scales = None
    assert call(d) == -1
    d.act.out.values = None                                    # copy-only needs its copy
    assert call(d) == -1
    d.act.out.normed = A16 + 64                                # copy over the input
    assert call(d) == -5


def test_binding_refuses_without_library(monkeypatch):
    """The binding fails loudly when libafq.so is missing (no fallback)."""
    monkeypatch.setattr(afq, "_lib", None)
    monkeypatch.setattr(afq, "library_path", "/nonexistent/libafq.so")
    with pytest.raises(ImportError):
        afq.load()
