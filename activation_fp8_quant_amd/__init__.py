"""activation_fp8_quant_amd -- fused activation FP8 quantisation for MI355X.

Thin Python binding over ``libafq.so`` (C ABI in ``include/afq.h``): it
allocates output tensors with PyTorch, marshals pointers and the current HIP
stream into the ABI descriptors, and raises on a non-zero status.  Every step
of the computation runs in the library's HIP kernels; there is no fallback.

Entry points (same names as the C ABI):
    fused_add_rmsnorm_quant(x, weight, eps, ...)   residual add + RMSNorm + quant
    silu_mul_quant(gate_up, mode, ...)             SiLU-and-mul + quant
    swiglu_oai_quant(gate_up, alpha, beta, limit)  clamped SwiGLU + MXFP8
    fp8_quant(x, mode, ...)                        standalone row-wise quant
and prepare(entry, *args, **kwargs): the arguments of one launch checked and
marshalled once, for eager loops that launch on the same buffers again.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import struct
import threading
from typing import Optional, Sequence, Union

import torch  # loaded first: the library then binds to torch's HIP runtime

__all__ = [
    "MXFP8", "BLOCK128", "PER_TOKEN", "STANDARD", "GEMMA",
    "QIN_DEFAULT", "QIN_FP32", "QIN_BF16",
    "QuantizedActivation", "AfqError", "PreparedLaunch", "prepare",
    "fused_add_rmsnorm_quant", "silu_mul_quant", "swiglu_oai_quant", "fp8_quant",
    "abi_version", "status_string", "library_path", "load",
]

# ---------------------------------------------------------------- constants
MXFP8, BLOCK128, PER_TOKEN = 0, 1, 2
STANDARD, GEMMA = 0, 1
# what the quantiser reads: the path's default, the fp32 normed value (norm,
# 1x128 / per-token), or the bf16-rounded activation (SiLU-and-mul, MXFP8)
QIN_DEFAULT, QIN_FP32, QIN_BF16 = 0, 1, 2
_BF16, _FP16, _FP32 = 0, 1, 2
_DTYPE_TAG = {torch.bfloat16: _BF16, torch.float16: _FP16, torch.float32: _FP32}
_NORM_DTYPE_TAG = {torch.bfloat16: _BF16, torch.float16: _FP16}
_MODE_NAMES = {"mxfp8": MXFP8, "mx": MXFP8, "block128": BLOCK128, "b128": BLOCK128,
               "per_token": PER_TOKEN, "pt": PER_TOKEN}
_KIND_NAMES = {"standard": STANDARD, "gemma": GEMMA}

_HERE = os.path.dirname(os.path.abspath(__file__))
library_path = os.path.join(_HERE, "libafq.so")


class AfqError(RuntimeError):
    """A non-zero status returned by libafq."""

    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: {status_string(status)} (status {status})")


# ------------------------------------------------------------ ABI structs
class _QAct(ctypes.Structure):
    _fields_ = [("values", ctypes.c_void_p), ("scales", ctypes.c_void_p),
                ("normed", ctypes.c_void_p)]


class _NormSeg(ctypes.Structure):
    _fields_ = [("x", ctypes.c_void_p), ("x_row_stride", ctypes.c_int64),
                ("weight", ctypes.c_void_p), ("cols", ctypes.c_int64), ("out", _QAct)]


class _NormDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("nseg", ctypes.c_int32), ("kind", ctypes.c_int32),
                ("dtype", ctypes.c_int32), ("mode", ctypes.c_int32), ("eps", ctypes.c_float),
                ("quant_input", ctypes.c_int32), ("residual_in", ctypes.c_void_p),
                ("residual_out", ctypes.c_void_p), ("seg", _NormSeg * 2)]


class _ActDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("I", ctypes.c_int64), ("gate_up", ctypes.c_void_p),
                ("gate_up_row_stride", ctypes.c_int64), ("mode", ctypes.c_int32),
                ("quant_input", ctypes.c_int32), ("out", _QAct)]


class _SwigluDesc(ctypes.Structure):
    _fields_ = [("act", _ActDesc), ("alpha", ctypes.c_float), ("beta", ctypes.c_float),
                ("limit", ctypes.c_float)]


class _QuantDesc(ctypes.Structure):
    _fields_ = [("M", ctypes.c_int64), ("cols", ctypes.c_int64), ("x", ctypes.c_void_p),
                ("x_row_stride", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("mode", ctypes.c_int32), ("out", _QAct)]


_lib = None


def load():
    """Load libafq.so (raises if it has not been built)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(library_path):
        raise ImportError(
            f"{library_path} is missing: build it with "
            "`python -m activation_fp8_quant_amd.build` (there is no fallback path)")
    lib = ctypes.CDLL(library_path)
    for name, desc in (("fused_add_rmsnorm_quant", _NormDesc), ("silu_mul_quant", _ActDesc),
                       ("swiglu_oai_quant", _SwigluDesc), ("fp8_quant", _QuantDesc)):
        f = getattr(lib, name)
        f.restype = ctypes.c_int
        f.argtypes = [ctypes.POINTER(desc), ctypes.c_void_p]
    lib.afq_status_string.restype = ctypes.c_char_p
    lib.afq_status_string.argtypes = [ctypes.c_int]
    lib.afq_abi_version.restype = ctypes.c_int
    lib.afq_abi_version.argtypes = []
    lib.afq_last_hip_error.restype = ctypes.c_int
    lib.afq_last_hip_error.argtypes = []
    _check_single_hip_runtime()
    _lib = lib
    return lib


def _check_single_hip_runtime():
    """The library must share torch's HIP runtime (one libamdhip64 mapped),
    otherwise torch's streams and pointers mean nothing to it."""
    try:
        with open("/proc/self/maps") as f:
            paths = {line.split()[-1] for line in f if "libamdhip64" in line}
    except OSError:
        return
    real = {os.path.realpath(p) for p in paths}
    if len(real) > 1:
        raise ImportError(f"two HIP runtimes are mapped: {sorted(real)}")


def abi_version() -> int:
    return load().afq_abi_version()


def status_string(status: int) -> str:
    return load().afq_status_string(int(status)).decode()


# ----------------------------------------------------------------- results
@dataclasses.dataclass(slots=True)
class QuantizedActivation:
    """Codes and scales of a quantised activation (the tuple a quantised
    linear consumes), with the optional rounded activation and residual.

    values   float8_e4m3fn [M, cols] (None for a copy-only launch)
    scales   MXFP8: uint8 E8M0 bytes [M, cols/32]; BLOCK128: float32
             [M, cols/128]; PER_TOKEN: float32 [M, 1] (None for a copy-only
             launch)
    normed   the rounded activation in its dtype, or None
    residual the updated residual h = x + r (norm with residual), or None
    """
    values: Optional[torch.Tensor]
    scales: Optional[torch.Tensor]
    normed: Optional[torch.Tensor]
    residual: Optional[torch.Tensor]
    mode: int
    orig_dtype: torch.dtype
    orig_shape: tuple


_MODES = {MXFP8: MXFP8, BLOCK128: BLOCK128, PER_TOKEN: PER_TOKEN}
_KINDS = {STANDARD: STANDARD, GEMMA: GEMMA}


def _mode(m) -> int:
    v = _MODES.get(m) if m.__class__ is int else None
    if v is not None:
        return v
    if isinstance(m, str):
        return _MODE_NAMES[m.lower()]
    if m not in (MXFP8, BLOCK128, PER_TOKEN):
        raise ValueError(f"unknown quant mode {m!r}")
    return int(m)


def _kind(k) -> int:
    v = _KINDS.get(k) if k.__class__ is int else None
    if v is not None:
        return v
    if isinstance(k, str):
        return _KIND_NAMES[k.lower()]
    if k not in (STANDARD, GEMMA):
        raise ValueError(f"unknown norm kind {k!r}")
    return int(k)


def _scales_shape(mode: int, M: int, cols: int):
    if mode == MXFP8:
        return (M, cols // 32), torch.uint8
    if mode == BLOCK128:
        return (M, cols // 128), torch.float32
    return (M, 1), torch.float32


def _ptr(t: Optional[torch.Tensor]):
    return 0 if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)
# the current device index without torch.cuda.current_device()'s wrapper
# (the tensors are already on a device, so the runtime is initialised)
_current_device = getattr(torch._C, "_cuda_getDevice", None) or torch.cuda.current_device


def _stream(stream, dev: int) -> int:
    """The HIP stream handle to enqueue on: the given stream, else torch's
    current stream on device index `dev` (the tensors' device)."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(dev)
        return torch.cuda.current_stream(dev).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _device_of(t: torch.Tensor, name: str) -> int:
    """The device index of a device tensor (raises for a host tensor)."""
    d = t.get_device()
    if d < 0:
        raise ValueError(f"{name} must be a device tensor")
    return d


def _rowmajor(t: torch.Tensor, name: str, dev: int):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if t.get_device() != dev:
        raise ValueError(f"{name} must be a device tensor on cuda:{dev}")


def _check_buf(t: torch.Tensor, numel: int, dtypes, dev: int, name: str):
    """A caller-supplied output: contiguous, on the inputs' device, of an
    accepted dtype and exactly the element count the kernel writes (the
    library takes raw pointers and cannot check extents itself)."""
    if t.get_device() != dev or t.dtype not in dtypes or t.numel() != numel or not t.is_contiguous():
        if t.get_device() != dev:
            raise ValueError(f"{name} must be a device tensor on cuda:{dev}")
        if t.dtype not in dtypes:
            raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
        raise ValueError(f"{name} must be a contiguous tensor of {numel} elements "
                         f"(got shape {tuple(t.shape)}, contiguous={t.is_contiguous()})")


_CODE_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def _alloc_out(mode, M, cols, dev: int, normed_dtype, want, out, quantize=True):
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a (values, scales, normed) tuple")
        values, scales, normed = out
        if not quantize:
            if values is not None or scales is not None or normed is None:
                raise ValueError("a copy-only launch takes out = (None, None, copy)")
            _check_buf(normed, M * cols, (normed_dtype,), dev, "out normed")
            return None, None, normed
        if values is None or scales is None:
            raise ValueError("out must give the values and scales buffers")
        _check_buf(values, M * cols, _CODE_DTYPES, dev, "out values")
        if mode == MXFP8:
            _check_buf(scales, M * (cols // 32), (torch.uint8,), dev, "out scales")
        else:
            _check_buf(scales, M * (cols // 128 if mode == BLOCK128 else 1), (torch.float32,), dev,
                       "out scales")
        if normed is not None:
            _check_buf(normed, M * cols, (normed_dtype,), dev, "out normed")
        return values, scales, normed
    if not quantize:
        return None, None, torch.empty((M, cols), dtype=normed_dtype, device=dev)
    sshape, sdtype = _scales_shape(mode, M, cols)
    values = torch.empty((M, cols), dtype=torch.float8_e4m3fn, device=dev)
    scales = torch.empty(sshape, dtype=sdtype, device=dev)
    normed = torch.empty((M, cols), dtype=normed_dtype, device=dev) if want else None
    return values, scales, normed


# ------------------------------------------------------ descriptor packing
# A call's descriptor is written with one struct.pack_into into a buffer
# that a ctypes view of the ABI struct shares (the format is derived from the
# ctypes layouts above, which tests/test_abi_cpu.py checks against the C
# header): far cheaper per call than setting the struct's fields one by one.
_CODES = {ctypes.c_int64: "q", ctypes.c_int32: "i", ctypes.c_float: "f", ctypes.c_void_p: "Q"}


def _leaves(cls, base=0):
    out = []
    for name, ftype in cls._fields_:
        off = base + getattr(cls, name).offset
        if isinstance(ftype, type) and issubclass(ftype, ctypes.Structure):
            out += _leaves(ftype, off)
        elif isinstance(ftype, type) and issubclass(ftype, ctypes.Array):
            et = ftype._type_
            for i in range(ftype._length_):
                out += _leaves(et, off + i * ctypes.sizeof(et))
        else:
            out.append((off, _CODES[ftype]))
    return out


def _packer(cls) -> struct.Struct:
    fmt, pos = "<", 0
    for off, code in sorted(_leaves(cls)):
        assert off >= pos
        fmt += "x" * (off - pos) + code
        pos = off + struct.calcsize("<" + code)
    fmt += "x" * (ctypes.sizeof(cls) - pos)
    packer = struct.Struct(fmt)
    assert packer.size == ctypes.sizeof(cls)
    return packer


_NORM_PACK = _packer(_NormDesc)    # M nseg kind dtype mode eps qin res_in res_out, 2 x (x stride w cols values scales normed)
_ACT_PACK = _packer(_ActDesc)      # M I gate_up stride mode qin values scales normed
_SWIGLU_PACK = _packer(_SwigluDesc)  # the _ActDesc fields, alpha beta limit
_QUANT_PACK = _packer(_QuantDesc)  # M cols x stride dtype mode values scales normed
_NO_SEG = (0,) * 7


class _Desc:
    """A descriptor buffer and the ctypes view the C call takes."""
    __slots__ = ("buf", "view", "ref")

    def __init__(self, cls):
        self.buf = bytearray(ctypes.sizeof(cls))
        self.view = cls.from_buffer(self.buf)
        self.ref = ctypes.byref(self.view)


class _PerThread(threading.local):
    """Per-thread descriptor buffers for immediate calls (the library reads
    a descriptor before it returns, so one buffer per entry point serves
    every call of a thread)."""

    def __init__(self):
        self.norm = _Desc(_NormDesc)
        self.act = _Desc(_ActDesc)
        self.swiglu = _Desc(_SwigluDesc)
        self.quant = _Desc(_QuantDesc)


_tls = _PerThread()


class PreparedLaunch:
    """One launch whose arguments were checked and marshalled into its C
    descriptor once.  Calling it enqueues the same launch again -- same input
    and output buffers, on the given stream (default: torch's current stream
    on the buffers' device) -- and returns the same result object, whose
    tensors the launch has overwritten.  It holds references to every buffer
    the descriptor points to; the caller must not resize them or change
    their storage (their contents may change freely between calls: the
    launch reads them when it runs)."""

    __slots__ = ("_fn", "_desc", "_dev", "result", "_keep", "_what")

    def __init__(self, fn, desc: _Desc, dev: int, result, keep, what: str):
        self._fn, self._desc, self._dev = fn, desc, dev
        self.result, self._keep, self._what = result, keep, what

    def __call__(self, stream=None):
        _call(self._fn, self._desc.ref, stream, self._dev, self._what)
        return self.result


def _call(fn, ref, stream, dev: int, what: str):
    """Call an entry point with the tensors' device current (HIP launches on
    the current device)."""
    arg = _stream(stream, dev)
    if dev != _current_device():
        with torch.cuda.device(dev):
            st = fn(ref, arg)
    else:
        st = fn(ref, arg)
    if st != 0:
        raise AfqError(st, what)


def _finish(fn, slot: str, packer: struct.Struct, fields, stream, dev: int, result, keep, what: str,
            defer: bool):
    """Pack the descriptor and launch now (returning the result), or hand
    back the prepared launch (with a descriptor buffer of its own)."""
    if defer:
        desc = _Desc({"norm": _NormDesc, "act": _ActDesc, "swiglu": _SwigluDesc,
                      "quant": _QuantDesc}[slot])
        packer.pack_into(desc.buf, 0, *fields)
        return PreparedLaunch(fn, desc, dev, result, keep, what)
    desc = getattr(_tls, slot)
    packer.pack_into(desc.buf, 0, *fields)
    _call(fn, desc.ref, stream, dev, what)
    return result


# ------------------------------------------------------------- entry points
def fused_add_rmsnorm_quant(
    x: Union[torch.Tensor, Sequence[torch.Tensor]],
    weight: Union[torch.Tensor, Sequence[torch.Tensor]],
    eps: float,
    *,
    mode=MXFP8,
    kind=GEMMA,
    residual: Optional[torch.Tensor] = None,
    residual_out: Optional[torch.Tensor] = None,
    inplace: bool = False,
    want_normed: bool = False,
    quant_input: int = QIN_DEFAULT,
    quantize: bool = True,
    out=None,
    stream=None,
    _defer: bool = False,
):
    """Residual add + RMSNorm + FP8 quantisation in one launch.

    x / weight   one [M, cols] tensor and its [cols] weight, or two of each
                 (two independent row segments, e.g. the q and kv inputs of
                 MLA attention, normed in one launch with separate weights)
    residual     [M, cols] or None.  The updated residual h = x + residual
                 goes to residual_out (a new tensor by default, `residual`
                 itself with inplace=True).
    want_normed  also return the normed rows rounded to the input dtype.
    quant_input  QIN_DEFAULT: quantise the dtype-rounded normed rows;
                 QIN_FP32 (1x128 / per-token): quantise the fp32 normed value.
    quantize     False: the norm of the unfused chain -- only the normed rows
                 (and the residual) are written; values and scales are None.
    out          optional preallocated (values, scales, normed) per segment
                 (a tuple, or a list of tuples for two segments).
    Returns a QuantizedActivation, or a list of two for two segments.
    """
    lib = _lib or load()
    mode, kind = _mode(mode), _kind(kind)
    if isinstance(x, torch.Tensor):
        if not isinstance(weight, torch.Tensor):
            raise ValueError("x and weight must both be one tensor or two tensors")
        return _norm_one(lib, x, weight, eps, mode, kind, residual, residual_out, inplace,
                         want_normed, quant_input, quantize, out, stream, _defer)
    else:
        xs = list(x)
        ws = [weight] if isinstance(weight, torch.Tensor) else list(weight)
        if len(xs) != len(ws) or len(xs) not in (1, 2):
            raise ValueError("x and weight must both be one tensor or two tensors")
        outs = [out] if (out is None or len(xs) == 1) else list(out)
        if len(outs) == 1 and len(xs) == 2:
            outs = [None, None]
    x0 = xs[0]
    dtype = x0.dtype
    dtag = _NORM_DTYPE_TAG.get(dtype)
    if dtag is None:
        raise TypeError("norm inputs must be bfloat16 or float16")
    dev = _device_of(x0, "x")
    M = x0.shape[0]
    fields = [M, len(xs), kind, dtag, mode, float(eps), int(quant_input), 0, 0]
    results = []
    for xi, wi, oi in zip(xs, ws, outs):
        _rowmajor(xi, "x", dev)
        if wi.get_device() != dev:
            raise ValueError(f"weight must be a device tensor on cuda:{dev}")
        if xi.dtype != dtype or wi.dtype != dtype or xi.shape[0] != M:
            raise ValueError("segments must share dtype and row count")
        cols = xi.shape[1]
        if wi.dim() != 1 or wi.shape[0] != cols or not wi.is_contiguous():
            raise ValueError("weight must be a contiguous [cols] tensor")
        values, scales, normed = _alloc_out(mode, M, cols, dev, dtype, want_normed, oi, quantize)
        fields += (xi.data_ptr(), xi.stride(0), wi.data_ptr(), cols,
                   _ptr(values), _ptr(scales), _ptr(normed))
        results.append(QuantizedActivation(values, scales, normed, None, mode, dtype, (M, cols)))
    if len(xs) == 1:
        fields += _NO_SEG
    if residual is not None:
        if len(xs) != 1:
            raise ValueError("a residual is only supported with one segment")
        _rowmajor(residual, "residual", dev)
        if not residual.is_contiguous() or residual.dtype != dtype or residual.shape != x0.shape:
            raise ValueError("residual must be a contiguous tensor shaped and typed like x")
        if residual_out is None:
            residual_out = residual if inplace else torch.empty_like(residual)
        else:
            _check_buf(residual_out, residual.numel(), (dtype,), dev, "residual_out")
        fields[7], fields[8] = residual.data_ptr(), residual_out.data_ptr()
        results[0].residual = residual_out
    elif residual_out is not None:
        raise ValueError("residual_out needs a residual")
    return _finish(lib.fused_add_rmsnorm_quant, "norm", _NORM_PACK, fields, stream, dev,
                   results[0] if len(results) == 1 else results, (xs, ws, residual),
                   "fused_add_rmsnorm_quant", _defer)


def _norm_one(lib, x, w, eps, mode, kind, residual, residual_out, inplace, want_normed, quant_input,
              quantize, out, stream, defer):
    """fused_add_rmsnorm_quant with one segment: the same checks and fields
    as the general path, written out for the per-call host cost."""
    dtype = x.dtype
    dtag = _NORM_DTYPE_TAG.get(dtype)
    if dtag is None:
        raise TypeError("norm inputs must be bfloat16 or float16")
    dev = x.get_device()
    if dev < 0:
        raise ValueError("x must be a device tensor")
    if x.dim() != 2 or x.stride(1) != 1:
        raise ValueError("x must be a 2-D tensor with unit column stride")
    M, cols = x.shape
    if w.get_device() != dev:
        raise ValueError(f"weight must be a device tensor on cuda:{dev}")
    if w.dtype != dtype or w.dim() != 1 or w.shape[0] != cols or not w.is_contiguous():
        raise ValueError("weight must be a contiguous [cols] tensor of the input dtype")
    values, scales, normed = _alloc_out(mode, M, cols, dev, dtype, want_normed, out, quantize)
    rin = rout = 0
    if residual is not None:
        if residual.get_device() != dev:
            raise ValueError(f"residual must be a device tensor on cuda:{dev}")
        if residual.dtype != dtype or residual.dim() != 2 or residual.shape[0] != M or \
                residual.shape[1] != cols or not residual.is_contiguous():
            raise ValueError("residual must be a contiguous tensor shaped and typed like x")
        if residual_out is None:
            residual_out = residual if inplace else torch.empty_like(residual)
        else:
            _check_buf(residual_out, M * cols, (dtype,), dev, "residual_out")
        rin, rout = residual.data_ptr(), residual_out.data_ptr()
    elif residual_out is not None:
        raise ValueError("residual_out needs a residual")
    fields = (M, 1, kind, dtag, mode, float(eps), int(quant_input), rin, rout,
              x.data_ptr(), x.stride(0), w.data_ptr(), cols,
              0 if values is None else values.data_ptr(), 0 if scales is None else scales.data_ptr(),
              0 if normed is None else normed.data_ptr()) + _NO_SEG
    qa = QuantizedActivation(values, scales, normed, residual_out, mode, dtype, (M, cols))
    return _finish(lib.fused_add_rmsnorm_quant, "norm", _NORM_PACK, fields, stream, dev, qa,
                   (x, w, residual), "fused_add_rmsnorm_quant", defer)


def _act_fields(gate_up, mode, want_act, quant_input, quantize, out):
    """Checks, output allocation and the descriptor fields shared by the
    SiLU-and-mul and clamped-SwiGLU entry points."""
    dev = _device_of(gate_up, "gate_up")
    _rowmajor(gate_up, "gate_up", dev)
    if gate_up.dtype != torch.bfloat16:
        raise TypeError("gate_up must be bfloat16")
    M, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up must have an even number of columns")
    I = two_i // 2
    values, scales, act = _alloc_out(mode, M, I, dev, torch.bfloat16, want_act, out, quantize)
    fields = (M, I, gate_up.data_ptr(), gate_up.stride(0), mode, int(quant_input),
              _ptr(values), _ptr(scales), _ptr(act))
    return dev, fields, QuantizedActivation(values, scales, act, None, mode, torch.bfloat16, (M, I))


def silu_mul_quant(gate_up: torch.Tensor, mode=MXFP8, *, want_act: bool = False,
                   quant_input: int = QIN_DEFAULT, quantize: bool = True, out=None,
                   stream=None, _defer: bool = False) -> QuantizedActivation:
    """SiLU-and-mul of a bf16 [M, 2I] row ([gate | up]) + FP8 quantisation.

    MXFP8 quantises the fp32 activation; BLOCK128 rounds silu and the product
    to bf16 first (the unfused SiluAndMul).  With MXFP8, quant_input=QIN_BF16
    quantises the bf16-rounded activation instead (the unfused chain's
    rounding).  want_act also returns the bf16 activation.  quantize=False:
    the SiLU-and-mul of the unfused chain -- only the bf16 activation (rounded
    as `mode` rounds it) is written; values and scales are None.
    """
    lib = _lib or load()
    mode = _mode(mode)
    dev, fields, qa = _act_fields(gate_up, mode, want_act, quant_input, quantize, out)
    return _finish(lib.silu_mul_quant, "act", _ACT_PACK, fields, stream, dev, qa, gate_up,
                   "silu_mul_quant", _defer)


def swiglu_oai_quant(gate_up: torch.Tensor, alpha: float, beta: float, limit: float, *,
                     want_act: bool = False, quant_input: int = QIN_DEFAULT,
                     quantize: bool = True, out=None, stream=None,
                     _defer: bool = False) -> QuantizedActivation:
    """Clamped SwiGLU of a bf16 [M, 2I] row ([gate | up]) + MXFP8:
    a = fp32(glu) * fp32(clamp(up, +-limit) + beta), glu = gc * logistic(alpha
    * gc), gc = min(gate, limit), quantised in fp32.  quant_input=QIN_BF16
    quantises the bf16-rounded activation; quantize=False writes only the bf16
    activation (the unfused chain's first kernel)."""
    lib = _lib or load()
    dev, fields, qa = _act_fields(gate_up, MXFP8, want_act, quant_input, quantize, out)
    return _finish(lib.swiglu_oai_quant, "swiglu", _SWIGLU_PACK,
                   fields + (float(alpha), float(beta), float(limit)), stream, dev, qa, gate_up,
                   "swiglu_oai_quant", _defer)


def fp8_quant(x: torch.Tensor, mode=MXFP8, *, out=None, stream=None,
              _defer: bool = False) -> QuantizedActivation:
    """Standalone row-wise FP8 quantisation of a bf16 / fp16 / fp32 [M, cols]."""
    lib = _lib or load()
    mode = _mode(mode)
    dev = _device_of(x, "x")
    _rowmajor(x, "x", dev)
    dtag = _DTYPE_TAG.get(x.dtype)
    if dtag is None:
        raise TypeError("x must be bfloat16, float16 or float32")
    M, cols = x.shape
    if out is not None and out[2] is not None:
        raise ValueError("fp8_quant writes no rounded copy: out[2] must be None")
    values, scales, _ = _alloc_out(mode, M, cols, dev, None, False, out)
    fields = (M, cols, x.data_ptr(), x.stride(0), dtag, mode, _ptr(values), _ptr(scales), 0)
    return _finish(lib.fp8_quant, "quant", _QUANT_PACK, fields, stream, dev,
                   QuantizedActivation(values, scales, None, None, mode, x.dtype, (M, cols)), x,
                   "fp8_quant", _defer)


def prepare(entry, *args, **kwargs) -> PreparedLaunch:
    """Check and marshal the arguments of one call of `entry` (one of
    fused_add_rmsnorm_quant, silu_mul_quant, swiglu_oai_quant, fp8_quant)
    without launching; the returned PreparedLaunch launches it.  Outputs not
    passed in `out` are allocated here, once, and reused by every call."""
    if entry not in (fused_add_rmsnorm_quant, silu_mul_quant, swiglu_oai_quant, fp8_quant):
        raise ValueError("prepare takes one of the library's entry points")
    if "stream" in kwargs:
        raise ValueError("pass the stream to the prepared launch, not to prepare")
    return entry(*args, _defer=True, **kwargs)


