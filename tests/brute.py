"""Exact brute-force reference for tiny rows (test infrastructure).

Independent of the C oracle: rationals (fractions.Fraction) for every exact
step, a 60-digit decimal square root and exponential for the two
irrational steps, and rounding to a format by enumerating every
representable value.  Slow (pure Python); rows of 32..128 elements.
"""
from __future__ import annotations

from decimal import Decimal, getcontext
from fractions import Fraction

import numpy as np

getcontext().prec = 60

_E4M3 = None
_BF16 = None
_FP16 = None


def _e4m3_values():
    """(value, code) of every non-negative finite e4m3fn code, from the
    field definition: bias 7, 3 mantissa bits, S.1111.111 = NaN."""
    global _E4M3
    if _E4M3 is None:
        out = []
        for c in range(0x7F):
            e, m = c >> 3, c & 7
            v = Fraction(m, 8) * Fraction(2) ** -6 if e == 0 else (1 + Fraction(m, 8)) * Fraction(2) ** (e - 7)
            out.append((v, c))
        _E4M3 = out
    return _E4M3


def _fmt_values(ebits, mbits, bias):
    out = []
    emax = (1 << ebits) - 1
    for e in range(emax):  # exponent all-ones is inf/nan
        for m in range(1 << mbits):
            if e == 0:
                v = Fraction(m, 1 << mbits) * Fraction(2) ** (1 - bias)
            else:
                v = (1 + Fraction(m, 1 << mbits)) * Fraction(2) ** (e - bias)
            out.append((v, (e << mbits) | m))
    return out


def _bf16_values():
    global _BF16
    if _BF16 is None:
        _BF16 = _fmt_values(8, 7, 127)
    return _BF16


def _fp16_values():
    global _FP16
    if _FP16 is None:
        _FP16 = _fmt_values(5, 10, 15)
    return _FP16


def nearest(v, table):
    """Nearest table value to real v (Fraction or Decimal), ties to the even
    code; returns (code with sign bit, value).  Binary search on the sorted
    table, then an exact comparison with the neighbours."""
    neg = v < 0
    a = -v if neg else v
    lo, hi = 0, len(table) - 1
    vals = _values_of(table)
    if a >= vals[-1]:
        i = len(table) - 1
    else:
        while hi - lo > 1:
            mid = (lo + hi) // 2
            if _le(vals[mid], a):
                lo = mid
            else:
                hi = mid
        d_lo = _absdiff(a, vals[lo])
        d_hi = _absdiff(a, vals[lo + 1])
        if d_lo < d_hi:
            i = lo
        elif d_hi < d_lo:
            i = lo + 1
        else:
            i = lo if table[lo][1] % 2 == 0 else lo + 1
    code, val = table[i][1], table[i][0]
    return code, (-val if neg else val)


_VALS = {}


def _values_of(table):
    k = id(table)
    if k not in _VALS:
        _VALS[k] = [t[0] for t in table]
    return _VALS[k]


def _le(f: Fraction, a) -> bool:
    if isinstance(a, Decimal):
        return Decimal(f.numerator) / Decimal(f.denominator) <= a
    return f <= a


def _absdiff(a, f: Fraction):
    if isinstance(a, Decimal):
        return abs(a - Decimal(f.numerator) / Decimal(f.denominator))
    return abs(a - f)


_BY_CODE = {}


def frac_of_bits16(b, dtype):
    if dtype not in _BY_CODE:
        table = _bf16_values() if dtype == "bf16" else _fp16_values()
        _BY_CODE[dtype] = dict((c, v) for v, c in table)
    b = int(b)
    val = _BY_CODE[dtype][b & 0x7FFF]
    return -val if b & 0x8000 else val


def round16(v, dtype):
    table = _bf16_values() if dtype == "bf16" else _fp16_values()
    code, val = nearest(v, table)
    sign = 0x8000 if v < 0 or (v == 0 and str(v).startswith("-")) else 0
    return code | sign, val


def e4m3(v: Fraction):
    """e4m3 code of an exact value already clamped to [-448, 448]."""
    code, _ = nearest(v, _e4m3_values())
    return code | (0x80 if v < 0 else 0)


def quant_mx(u):
    """u: list of Fraction (a 32-block).  Returns (codes, byte)."""
    amax = max(abs(x) for x in u)
    if amax == 0:
        b = 0
    else:
        # smallest b with amax / 2^(b-127) < 512
        b = next(b for b in range(255) if amax / Fraction(2) ** (b - 127) < 512)
    X = Fraction(2) ** (b - 127)
    codes = []
    for x in u:
        v = x / X
        v = max(min(v, Fraction(448)), Fraction(-448))
        c = e4m3(v)
        if x == 0 and c == 0:
            c = 0
        codes.append(c)
    return codes, b


def quant_fp32scale(u):
    """u: list of Fraction (one group); fp32 arithmetic for the stored scale
    and the quotient (numpy float32 division is IEEE)."""
    amax = max(abs(x) for x in u)
    A = np.float32(float(amax))
    s = np.float32(A / np.float32(448.0))
    if s == 0:          # all zero, or amax / 448 below half the least subnormal
        return [0] * len(u), s
    codes = []
    for x in u:
        t = np.float32(np.float32(float(x)) / s)
        v = Fraction(float(t))
        v = max(min(v, Fraction(448)), Fraction(-448))
        codes.append(e4m3(v) if v != 0 else (0x80 if np.signbit(t) else 0))
    return codes, s


def rn_f32(v) -> Fraction:
    """The fp32 value nearest to the exact value v (Fraction or Decimal),
    ties to even significand; subnormals included, no overflow expected."""
    v = Fraction(v)
    if v == 0:
        return v
    a = abs(v)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    e = max(e, -126)                      # below 2^-126 the quantum is fixed
    q = Fraction(2) ** (e - 23)
    n = a / q
    k = n.numerator // n.denominator
    rem = n - k
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and k % 2 == 1):
        k += 1
    return k * q if v > 0 else -k * q


def norm_row(x_bits, r_bits, w_bits, kind, dtype, mode, eps, qin="default"):
    """One row: returns dict(h, normed, codes, scales) as python ints /
    numpy float32 scales.  qin = "fp32": the fp32-direct variant, whose
    quantiser reads y = fl32(fl32(h * fl32(inv)) * fl32(g)) (each step one
    exact rounding to fp32) and whose copy is that y rounded to the dtype."""
    H = len(x_bits)
    x = [frac_of_bits16(b, dtype) for b in x_bits]
    w = [frac_of_bits16(b, dtype) for b in w_bits]
    if r_bits is not None:
        r = [frac_of_bits16(b, dtype) for b in r_bits]
        hb = [round16(a + b, dtype) for a, b in zip(x, r)]
        h_codes = [c for c, _ in hb]
        h = [v for _, v in hb]
    else:
        h_codes, h = None, x
    ms = sum(v * v for v in h) / H
    den = Decimal(ms.numerator) / Decimal(ms.denominator) + Decimal(float(np.float32(eps)))
    inv = 1 / den.sqrt()
    u_codes, u = [], []
    if qin == "fp32":
        inv32 = rn_f32(inv)
        for hv, wv in zip(h, w):
            g32 = rn_f32(1 + wv) if kind == "gemma" else wv
            y = rn_f32(rn_f32(hv * inv32) * g32)
            c, _ = round16(y, dtype)
            u_codes.append(c)
            u.append(y)
    else:
        for hv, wv in zip(h, w):
            g = (1 + wv) if kind == "gemma" else wv
            y = Decimal(hv.numerator) / Decimal(hv.denominator) * inv * (Decimal(g.numerator) / Decimal(g.denominator))
            c, val = round16(y, dtype)
            u_codes.append(c)
            u.append(val)
    codes, scales = [], []
    G = 32 if mode == "mx" else 128 if mode == "b128" else H
    for k in range(0, H, G):
        if mode == "mx":
            q, s = quant_mx(u[k:k + G])
        else:
            q, s = quant_fp32scale(u[k:k + G])
        codes += q
        scales.append(s)
    return dict(h=h_codes, normed=u_codes, codes=codes, scales=scales)
