"""CPU oracle for fused activation FP8 quantisation -- TEST INFRASTRUCTURE.

Only the tests, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  The product path (the HIP library and
its Python binding) never does, and shares no code with it.

The arithmetic lives in ``afq_oracle.c`` (plain C, fp64, formats decoded from
their field definitions); this module only marshals numpy arrays into it.
bf16 and fp16 arrays are carried as ``uint16`` bit patterns, fp32 as
``float32``, e4m3 codes and E8M0 scale bytes as ``uint8``.
"""
from __future__ import annotations

import ctypes
import os
import threading

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_LIB_PATH = os.path.join(_HERE, "libafq_oracle.so")
_SRC_PATH = os.path.join(_HERE, "afq_oracle.c")

# enum values of afq_oracle.c
MXFP8, BLOCK128, PER_TOKEN = 0, 1, 2
BF16, FP16, FP32 = 0, 1, 2
STANDARD, GEMMA = 0, 1
# what the quantiser reads: the path's default, the fp32 normed value (norm,
# fp32-direct), or the bf16-rounded fp32 activation (MXFP8 SiLU, bf16-first)
QIN_DEFAULT, QIN_FP32, QIN_BF16 = 0, 1, 2

GROUP = {MXFP8: 32, BLOCK128: 128}

_lib = None
_lock = threading.Lock()


def build(force: bool = False) -> str:
    """Compile the oracle with gcc (-O2, no fast-math, no FP contraction)."""
    import subprocess

    if force or not os.path.exists(_LIB_PATH) or (
        os.path.getmtime(_LIB_PATH) < os.path.getmtime(_SRC_PATH)
    ):
        subprocess.check_call(
            ["gcc", "-O2", "-std=c11", "-fPIC", "-shared", "-ffp-contract=off",
             "-o", _LIB_PATH, _SRC_PATH, "-lm", "-lpthread"])
    return _LIB_PATH


def lib():
    global _lib
    with _lock:
        if _lib is None:
            build()
            L = ctypes.CDLL(_LIB_PATH)
            P, I64, I32, F32, D = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_int,
                                   ctypes.c_float, ctypes.c_double)
            L.orc_round_bf16.restype = ctypes.c_uint16
            L.orc_round_bf16.argtypes = [D]
            L.orc_round_fp16.restype = ctypes.c_uint16
            L.orc_round_fp16.argtypes = [D]
            L.orc_round_e4m3.restype = ctypes.c_uint8
            L.orc_round_e4m3.argtypes = [D]
            L.orc_e8m0_byte.restype = ctypes.c_uint8
            L.orc_e8m0_byte.argtypes = [F32]
            L.orc_silu.restype = D
            L.orc_silu.argtypes = [D]
            for name in ("orc_decode_bf16", "orc_decode_fp16"):
                getattr(L, name).restype = D
                getattr(L, name).argtypes = [ctypes.c_uint16]
            L.orc_decode_e4m3.restype = D
            L.orc_decode_e4m3.argtypes = [ctypes.c_uint8]
            for name in ("orc_round_bf16_n", "orc_round_fp16_n", "orc_round_e4m3_n",
                         "orc_e8m0_byte_n", "orc_silu_n"):
                getattr(L, name).restype = None
                getattr(L, name).argtypes = [P, P, I64]
            L.orc_quant_rows.restype = I32
            L.orc_quant_rows.argtypes = [I64, I64, P, I64, I32, I32, P, P, I64, I64, P]
            L.orc_norm_quant_rows.restype = I32
            L.orc_norm_quant_rows.argtypes = [I64, I64, P, I64, P, P, P, I32, I32, I32, I32,
                                              F32, P, P, P, I64, I64, P]
            L.orc_silu_quant_rows.restype = I32
            L.orc_silu_quant_rows.argtypes = [I64, I64, P, I64, I32, I32, P, P, P, I64, I64, P]
            L.orc_swiglu_glu32_n.restype = None
            L.orc_swiglu_glu32_n.argtypes = [P, P, I64, F32, F32]
            L.orc_swiglu_act32_n.restype = None
            L.orc_swiglu_act32_n.argtypes = [P, P, P, I64, F32, F32, F32]
            L.orc_swiglu_oai_quant_rows.restype = I32
            L.orc_swiglu_oai_quant_rows.argtypes = [I64, I64, P, I64, I32, I32, F32, F32, F32,
                                                    P, P, P, I64, I64, P]
            _lib = L
    return _lib


def _ptr(a):
    return None if a is None else a.ctypes.data


def _c(a, dtype):
    a = np.asarray(a)
    assert a.dtype == dtype, (a.dtype, dtype)
    return a


def _parallel_rows(M, threads, fn):
    """Run fn(r0, r1) over row ranges on `threads` Python threads (ctypes
    releases the GIL for the duration of each C call)."""
    threads = max(1, min(int(threads), int(M))) if M > 0 else 1
    if threads == 1:
        fn(0, M)
        return
    bounds = np.linspace(0, M, threads + 1).astype(np.int64)
    ts = [threading.Thread(target=fn, args=(int(bounds[k]), int(bounds[k + 1])))
          for k in range(threads)]
    for t in ts:
        t.start()
    for t in ts:
        t.join()


# ---------------------------------------------------------------- elementwise
def round_bf16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_round_bf16_n(_ptr(v), _ptr(out), v.size)
    return out


def round_fp16(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint16)
    lib().orc_round_fp16_n(_ptr(v), _ptr(out), v.size)
    return out


def round_e4m3(v) -> np.ndarray:
    v = np.ascontiguousarray(v, dtype=np.float64)
    out = np.empty(v.shape, np.uint8)
    lib().orc_round_e4m3_n(_ptr(v), _ptr(out), v.size)
    return out


def e8m0_byte(amax) -> np.ndarray:
    a = np.ascontiguousarray(amax, dtype=np.float32)
    out = np.empty(a.shape, np.uint8)
    lib().orc_e8m0_byte_n(_ptr(a), _ptr(out), a.size)
    return out


def silu(g) -> np.ndarray:
    g = np.ascontiguousarray(g, dtype=np.float64)
    out = np.empty(g.shape, np.float64)
    lib().orc_silu_n(_ptr(g), _ptr(out), g.size)
    return out


def swiglu_glu32(g, alpha: float, limit: float) -> np.ndarray:
    """fl32(min(g, limit) * logistic(alpha * min(g, limit))), alpha and limit
    taken as fp32 values: the gate factor of the clamped SwiGLU."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    out = np.empty(g.shape, np.float32)
    lib().orc_swiglu_glu32_n(_ptr(g), _ptr(out), g.size, float(alpha), float(limit))
    return out


def swiglu_act32(g, u, alpha: float, beta: float, limit: float) -> np.ndarray:
    """The fp32 clamped-SwiGLU activation fl32(glu32 * fl32(clamp(u) + beta))."""
    g = np.ascontiguousarray(g, dtype=np.float64)
    u = np.ascontiguousarray(u, dtype=np.float64)
    assert g.shape == u.shape
    out = np.empty(g.shape, np.float32)
    lib().orc_swiglu_act32_n(_ptr(g), _ptr(u), _ptr(out), g.size, float(alpha), float(beta),
                             float(limit))
    return out


def decode_bf16(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint16)
    return np.vectorize(lambda x: lib().orc_decode_bf16(int(x)), otypes=[np.float64])(c)


def decode_e4m3(c) -> np.ndarray:
    c = np.asarray(c, dtype=np.uint8)
    return np.vectorize(lambda x: lib().orc_decode_e4m3(int(x)), otypes=[np.float64])(c)


def _scales_array(M, n, mode):
    if mode == MXFP8:
        return np.zeros((M, n // 32), np.uint8)
    if mode == BLOCK128:
        return np.zeros((M, n // 128), np.float32)
    return np.zeros((M, 1), np.float32)


# ------------------------------------------------------------------ row ops
def quant(x, in_dtype: int, mode: int, threads: int = 1):
    """Standalone row-wise quantisation of x [M, n] -> (codes u8 [M, n], scales)."""
    x = np.ascontiguousarray(x)
    M, n = x.shape
    values = np.zeros((M, n), np.uint8)
    scales = _scales_array(M, n, mode)

    def run(r0, r1):
        work = np.empty(max(n, 1), np.float64)
        rc = lib().orc_quant_rows(M, n, _ptr(x), n, in_dtype, mode, _ptr(values),
                                  _ptr(scales), r0, r1, _ptr(work))
        assert rc == 0

    _parallel_rows(M, threads, run)
    return values, scales


def norm_quant(x, weight, *, residual=None, kind: int, dtype: int, mode: int,
               eps: float, want_normed: bool = True, threads: int = 1,
               rows=None, qin: int = QIN_DEFAULT):
    """(residual add +) RMSNorm + quantisation of x [M, H] (uint16 bit patterns).

    Returns dict(h=[M,H] u16 or None, values=[M,H] u8, scales, normed=u16 or None).
    `rows` optionally restricts the computation to a sorted index array of rows
    (the other rows of every output are left zero).  qin = QIN_FP32 quantises
    the fp32 normed value instead of the dtype-rounded row (fp32-direct).
    """
    x = np.ascontiguousarray(x, dtype=np.uint16)
    weight = np.ascontiguousarray(weight, dtype=np.uint16)
    M, H = x.shape
    assert weight.shape == (H,)
    if residual is not None:
        residual = np.ascontiguousarray(residual, dtype=np.uint16)
        assert residual.shape == (M, H)
        h = np.zeros((M, H), np.uint16)
    else:
        h = None
    values = np.zeros((M, H), np.uint8)
    scales = _scales_array(M, H, mode)
    normed = np.zeros((M, H), np.uint16) if want_normed else None

    def run_range(r0, r1):
        work = np.empty(2 * max(H, 1), np.float64)
        rc = lib().orc_norm_quant_rows(M, H, _ptr(x), H, _ptr(residual), _ptr(h),
                                       _ptr(weight), kind, dtype, mode, qin, float(eps),
                                       _ptr(values), _ptr(scales), _ptr(normed),
                                       r0, r1, _ptr(work))
        assert rc == 0

    if rows is None:
        _parallel_rows(M, threads, run_range)
    else:
        rows = np.asarray(rows, dtype=np.int64)
        work = np.empty(2 * max(H, 1), np.float64)
        for r in rows:
            rc = lib().orc_norm_quant_rows(M, H, _ptr(x), H, _ptr(residual), _ptr(h),
                                           _ptr(weight), kind, dtype, mode, qin, float(eps),
                                           _ptr(values), _ptr(scales), _ptr(normed),
                                           int(r), int(r) + 1, _ptr(work))
            assert rc == 0
    return dict(h=h, values=values, scales=scales, normed=normed)


def silu_quant(gu, mode: int, *, want_act: bool = True, threads: int = 1, rows=None,
               qin: int = QIN_DEFAULT):
    """SiLU-and-mul + quantisation of gu [M, 2I] bf16 ([gate | up]).  With
    MXFP8, qin = QIN_BF16 quantises the bf16-rounded activation (bf16-first)."""
    gu = np.ascontiguousarray(gu, dtype=np.uint16)
    M, two_i = gu.shape
    assert two_i % 2 == 0
    I = two_i // 2
    values = np.zeros((M, I), np.uint8)
    scales = _scales_array(M, I, mode)
    act = np.zeros((M, I), np.uint16) if want_act else None

    def run_range(r0, r1):
        work = np.empty(max(I, 1), np.float64)
        rc = lib().orc_silu_quant_rows(M, I, _ptr(gu), two_i, mode, qin, _ptr(values),
                                       _ptr(scales), _ptr(act), r0, r1, _ptr(work))
        if rc != 0:
            raise ValueError("oracle: SiLU-and-mul supports the MXFP8 and 1x128 modes")

    if rows is None:
        _parallel_rows(M, threads, run_range)
    else:
        for r in np.asarray(rows, dtype=np.int64):
            run_range(int(r), int(r) + 1)
    return dict(values=values, scales=scales, act=act)


def swiglu_oai_quant(gu, alpha: float, beta: float, limit: float, mode: int = MXFP8, *,
                     want_act: bool = True, threads: int = 1, rows=None,
                     qin: int = QIN_DEFAULT):
    """Clamped SwiGLU + MXFP8 quantisation of gu [M, 2I] bf16 ([gate | up]):
    a = fl32(fl32(glu) * fl32(clamp(up, +-limit) + beta)), glu =
    min(gate, limit) * logistic(alpha * min(gate, limit)).  qin = QIN_BF16
    quantises the bf16-rounded activation (the unfused chain's input)."""
    gu = np.ascontiguousarray(gu, dtype=np.uint16)
    M, two_i = gu.shape
    assert two_i % 2 == 0
    I = two_i // 2
    values = np.zeros((M, I), np.uint8)
    scales = _scales_array(M, I, mode)
    act = np.zeros((M, I), np.uint16) if want_act else None

    def run_range(r0, r1):
        work = np.empty(max(I, 1), np.float64)
        rc = lib().orc_swiglu_oai_quant_rows(M, I, _ptr(gu), two_i, mode, qin, float(alpha),
                                             float(beta), float(limit), _ptr(values),
                                             _ptr(scales), _ptr(act), r0, r1, _ptr(work))
        if rc != 0:
            raise ValueError("oracle: the clamped SwiGLU supports the MXFP8 mode only")

    if rows is None:
        _parallel_rows(M, threads, run_range)
    else:
        for r in np.asarray(rows, dtype=np.int64):
            run_range(int(r), int(r) + 1)
    return dict(values=values, scales=scales, act=act)
