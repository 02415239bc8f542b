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
@dataclasses.dataclass
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


def _mode(m) -> int:
    if isinstance(m, str):
        return _MODE_NAMES[m.lower()]
    if m not in (MXFP8, BLOCK128, PER_TOKEN):
        raise ValueError(f"unknown quant mode {m!r}")
    return int(m)


def _kind(k) -> int:
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
    return None if t is None else t.data_ptr()


_raw_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device: torch.device) -> int:
    """The HIP stream handle to enqueue on: the given stream, else torch's
    current stream on the tensors' device."""
    if stream is None:
        if _raw_stream is not None:
            return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())
        return torch.cuda.current_stream(device).cuda_stream
    if isinstance(stream, torch.cuda.Stream):
        return stream.cuda_stream
    return int(stream)


def _rowmajor(t: torch.Tensor, name: str):
    if t.dim() != 2 or t.stride(1) != 1:
        raise ValueError(f"{name} must be a 2-D tensor with unit column stride")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")


def _same_device(t: torch.Tensor, device: torch.device, name: str):
    if not t.is_cuda or t.device != device:
        raise ValueError(f"{name} must be a device tensor on {device}")


def _check_buf(t: torch.Tensor, numel: int, dtypes, device: torch.device, name: str):
    """A caller-supplied output: contiguous, on the inputs' device, of an
    accepted dtype and exactly the element count the kernel writes (the
    library takes raw pointers and cannot check extents itself)."""
    _same_device(t, device, name)
    if t.dtype not in dtypes:
        raise ValueError(f"{name} must have dtype {' or '.join(str(d) for d in dtypes)}, got {t.dtype}")
    if not t.is_contiguous() or t.numel() != numel:
        raise ValueError(f"{name} must be a contiguous tensor of {numel} elements "
                         f"(got shape {tuple(t.shape)}, contiguous={t.is_contiguous()})")


_CODE_DTYPES = (torch.float8_e4m3fn, torch.uint8)


def _alloc_out(mode, M, cols, device, normed_dtype, want, out, quantize=True):
    sshape, sdtype = _scales_shape(mode, M, cols)
    if out is not None:
        if len(out) != 3:
            raise ValueError("out must be a (values, scales, normed) tuple")
        values, scales, normed = out
        if not quantize:
            if values is not None or scales is not None or normed is None:
                raise ValueError("a copy-only launch takes out = (None, None, copy)")
            _check_buf(normed, M * cols, (normed_dtype,), device, "out normed")
            return None, None, normed
        _check_buf(values, M * cols, _CODE_DTYPES, device, "out values")
        _check_buf(scales, sshape[0] * sshape[1], (sdtype,), device, "out scales")
        if normed is not None:
            _check_buf(normed, M * cols, (normed_dtype,), device, "out normed")
        return values, scales, normed
    if not quantize:
        return None, None, torch.empty((M, cols), dtype=normed_dtype, device=device)
    values = torch.empty((M, cols), dtype=torch.float8_e4m3fn, device=device)
    scales = torch.empty(sshape, dtype=sdtype, device=device)
    normed = torch.empty((M, cols), dtype=normed_dtype, device=device) if want else None
    return values, scales, normed


class PreparedLaunch:
    """One launch whose arguments were checked and marshalled into its C
    descriptor once.  Calling it enqueues the same launch again -- same input
    and output buffers, on the given stream (default: torch's current stream
    on the buffers' device) -- and returns the same result object, whose
    tensors the launch has overwritten.  It holds references to every buffer
    the descriptor points to; the caller must not resize them or change
    their storage (their contents may change freely between calls: the
    launch reads them when it runs)."""

    __slots__ = ("_fn", "_desc", "_ref", "_device", "_index", "result", "_keep", "_what")

    def __init__(self, fn, desc, device: torch.device, result, keep, what: str):
        self._fn, self._desc, self._device = fn, desc, device
        self._ref = ctypes.byref(desc)
        self._index = device.index
        self.result, self._keep, self._what = result, keep, what

    def __call__(self, stream=None):
        arg = ctypes.c_void_p(_stream(stream, self._device))
        if self._index is not None and self._index != torch.cuda.current_device():
            with torch.cuda.device(self._device):
                st = self._fn(self._ref, arg)
        else:
            st = self._fn(self._ref, arg)
        if st != 0:
            raise AfqError(st, self._what)
        return self.result


def _finish(fn, desc, stream, device: torch.device, result, keep, what: str, defer: bool):
    """Launch now (returning the result), or hand back the prepared launch."""
    call = PreparedLaunch(fn, desc, device, result, keep, what)
    if defer:
        return call
    call(stream)
    return result


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
    lib = load()
    mode, kind = _mode(mode), _kind(kind)
    xs = [x] if isinstance(x, torch.Tensor) else list(x)
    ws = [weight] if isinstance(weight, torch.Tensor) else list(weight)
    if len(xs) != len(ws) or len(xs) not in (1, 2):
        raise ValueError("x and weight must both be one tensor or two tensors")
    outs = [out] if (out is None or len(xs) == 1) else list(out)
    if len(outs) == 1 and len(xs) == 2:
        outs = [None, None]
    dtype = xs[0].dtype
    if dtype not in (torch.bfloat16, torch.float16):
        raise TypeError("norm inputs must be bfloat16 or float16")
    M = xs[0].shape[0]
    _rowmajor(xs[0], "x")
    device = xs[0].device
    d = _NormDesc()
    d.M, d.nseg, d.kind, d.dtype, d.mode = M, len(xs), kind, _DTYPE_TAG[dtype], mode
    d.eps = float(eps)
    d.quant_input = int(quant_input)
    results = []
    for i, (xi, wi) in enumerate(zip(xs, ws)):
        _rowmajor(xi, "x")
        _same_device(xi, device, "x")
        _same_device(wi, device, "weight")
        if xi.dtype != dtype or wi.dtype != dtype or xi.shape[0] != M:
            raise ValueError("segments must share dtype and row count")
        if wi.dim() != 1 or wi.shape[0] != xi.shape[1] or not wi.is_contiguous():
            raise ValueError("weight must be a contiguous [cols] tensor")
        cols = xi.shape[1]
        values, scales, normed = _alloc_out(mode, M, cols, device, dtype, want_normed, outs[i],
                                            quantize)
        seg = d.seg[i]
        seg.x, seg.x_row_stride, seg.weight, seg.cols = xi.data_ptr(), xi.stride(0), wi.data_ptr(), cols
        seg.out.values, seg.out.scales, seg.out.normed = _ptr(values), _ptr(scales), _ptr(normed)
        results.append(QuantizedActivation(values, scales, normed, None, mode, dtype, tuple(xi.shape)))
    if residual is not None:
        if len(xs) != 1:
            raise ValueError("a residual is only supported with one segment")
        _rowmajor(residual, "residual")
        _same_device(residual, device, "residual")
        if not residual.is_contiguous() or residual.dtype != dtype or residual.shape != xs[0].shape:
            raise ValueError("residual must be a contiguous tensor shaped and typed like x")
        if residual_out is None:
            residual_out = residual if inplace else torch.empty_like(residual)
        else:
            _check_buf(residual_out, residual.numel(), (dtype,), device, "residual_out")
        d.residual_in, d.residual_out = residual.data_ptr(), residual_out.data_ptr()
        results[0].residual = residual_out
    elif residual_out is not None:
        raise ValueError("residual_out needs a residual")
    keep = (xs, ws, residual)
    return _finish(lib.fused_add_rmsnorm_quant, d, stream, device,
                   results[0] if len(results) == 1 else results, keep, "fused_add_rmsnorm_quant",
                   _defer)


def _act_desc(gate_up, mode, want_act, quant_input, quantize, out):
    """Checks, output allocation and the descriptor shared by the SiLU-and-mul
    and clamped-SwiGLU entry points."""
    _rowmajor(gate_up, "gate_up")
    if gate_up.dtype != torch.bfloat16:
        raise TypeError("gate_up must be bfloat16")
    M, two_i = gate_up.shape
    if two_i % 2:
        raise ValueError("gate_up must have an even number of columns")
    I = two_i // 2
    values, scales, act = _alloc_out(mode, M, I, gate_up.device, torch.bfloat16, want_act, out,
                                     quantize)
    d = _ActDesc()
    d.M, d.I, d.gate_up, d.gate_up_row_stride, d.mode = M, I, gate_up.data_ptr(), gate_up.stride(0), mode
    d.quant_input = int(quant_input)
    d.out.values, d.out.scales, d.out.normed = _ptr(values), _ptr(scales), _ptr(act)
    return d, QuantizedActivation(values, scales, act, None, mode, gate_up.dtype, (M, I))


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
    lib = load()
    mode = _mode(mode)
    d, qa = _act_desc(gate_up, mode, want_act, quant_input, quantize, out)
    return _finish(lib.silu_mul_quant, d, stream, gate_up.device, qa, gate_up, "silu_mul_quant",
                   _defer)


def swiglu_oai_quant(gate_up: torch.Tensor, alpha: float, beta: float, limit: float, *,
                     want_act: bool = False, quant_input: int = QIN_DEFAULT,
                     quantize: bool = True, out=None, stream=None,
                     _defer: bool = False) -> QuantizedActivation:
    """Clamped SwiGLU of a bf16 [M, 2I] row ([gate | up]) + MXFP8:
    a = fp32(glu) * fp32(clamp(up, +-limit) + beta), glu = gc * logistic(alpha
    * gc), gc = min(gate, limit), quantised in fp32.  quant_input=QIN_BF16
    quantises the bf16-rounded activation; quantize=False writes only the bf16
    activation (the unfused chain's first kernel)."""
    lib = load()
    d, qa = _act_desc(gate_up, MXFP8, want_act, quant_input, quantize, out)
    sd = _SwigluDesc()
    sd.act, sd.alpha, sd.beta, sd.limit = d, float(alpha), float(beta), float(limit)
    return _finish(lib.swiglu_oai_quant, sd, stream, gate_up.device, qa, gate_up,
                   "swiglu_oai_quant", _defer)


def fp8_quant(x: torch.Tensor, mode=MXFP8, *, out=None, stream=None,
              _defer: bool = False) -> QuantizedActivation:
    """Standalone row-wise FP8 quantisation of a bf16 / fp16 / fp32 [M, cols]."""
    lib = load()
    mode = _mode(mode)
    _rowmajor(x, "x")
    if x.dtype not in _DTYPE_TAG:
        raise TypeError("x must be bfloat16, float16 or float32")
    M, cols = x.shape
    if out is not None and out[2] is not None:
        raise ValueError("fp8_quant writes no rounded copy: out[2] must be None")
    values, scales, _ = _alloc_out(mode, M, cols, x.device, None, False, out)
    d = _QuantDesc()
    d.M, d.cols, d.x, d.x_row_stride = M, cols, x.data_ptr(), x.stride(0)
    d.dtype, d.mode = _DTYPE_TAG[x.dtype], mode
    d.out.values, d.out.scales, d.out.normed = _ptr(values), _ptr(scales), None
    return _finish(lib.fp8_quant, d, stream, x.device,
                   QuantizedActivation(values, scales, None, None, mode, x.dtype, (M, cols)), x,
                   "fp8_quant", _defer)
