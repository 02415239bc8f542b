"""Pins of the oracle's number formats against independent definitions:
library casts (torch / numpy), exact rational arithmetic, and closed values
of the OCP e4m3fn and E8M0 formats."""
from fractions import Fraction
import math

import numpy as np
import pytest
import torch

import oracle as orc


def _rng(seed=0):
    return np.random.default_rng(seed)


# ----------------------------------------------------------- decode tables
def test_decode_bf16_all_codes_match_torch():
    codes = np.arange(1 << 16, dtype=np.uint32)
    finite = ((codes >> 7) & 0xFF) != 0xFF
    c = codes[finite].astype(np.uint16)
    ref = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).double().numpy()
    got = np.array([orc.lib().orc_decode_bf16(int(x)) for x in c])
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


def test_decode_e4m3_all_codes_match_torch():
    c = np.array([x for x in range(256) if (x & 0x7F) != 0x7F], dtype=np.uint8)
    ref = torch.from_numpy(c).view(torch.float8_e4m3fn).double().numpy()
    got = np.array([orc.lib().orc_decode_e4m3(int(x)) for x in c])
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))
    assert orc.lib().orc_decode_e4m3(0x7E) == 448.0
    assert orc.lib().orc_decode_e4m3(0x01) == 2.0 ** -9
    assert orc.lib().orc_decode_e4m3(0x08) == 2.0 ** -6


def test_decode_fp16_all_codes_match_numpy():
    codes = np.arange(1 << 16, dtype=np.uint32)
    finite = ((codes >> 10) & 0x1F) != 0x1F
    c = codes[finite].astype(np.uint16)
    ref = c.view(np.float16).astype(np.float64)
    got = np.array([orc.lib().orc_decode_fp16(int(x)) for x in c])
    assert np.array_equal(got.view(np.uint64), ref.view(np.uint64))


# --------------------------------------------------------------- rounding
def _boundary_f32(rng, low_patterns):
    """fp32 values with every exponent, random high mantissa bits and the
    given low-bit patterns (where round-to-nearest decisions are made)."""
    exps = np.arange(0, 255, dtype=np.uint32)
    hi = rng.integers(0, 1 << 7, size=(exps.size, 8), dtype=np.uint32)
    out = []
    for lp in low_patterns:
        bits = (exps[:, None] << 23) | (hi << 16) | np.uint32(lp)
        out.append(bits.ravel())
    bits = np.concatenate(out)
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    return bits.view(np.float32)


def test_round_bf16_matches_torch_on_fp32():
    rng = _rng(1)
    v = np.concatenate([
        _boundary_f32(rng, [0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x18000]),
        (rng.standard_normal(200_000) * 10.0 ** rng.integers(-30, 30, 200_000)).astype(np.float32),
    ])
    v = v[np.abs(v) < 3.3e38]  # bf16 overflow handled separately
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    got = orc.round_bf16(v.astype(np.float64))
    assert np.array_equal(got, ref)


def test_round_fp16_matches_numpy_on_fp64():
    rng = _rng(2)
    v = np.concatenate([
        rng.standard_normal(200_000) * 10.0 ** rng.integers(-8, 5, 200_000),
        np.array([65504.0, 65519.99, -65519.0, 2.0 ** -24, 2.0 ** -25, 3 * 2.0 ** -26, -0.0, 0.0]),
    ])
    ref = v.astype(np.float16).view(np.uint16)
    got = orc.round_fp16(v)
    assert np.array_equal(got, ref)


def _nearest_exact(v: Fraction, values, codes):
    """Brute force: nearest of an enumerated value list, ties to even code."""
    best = None
    for val, code in zip(values, codes):
        d = abs(v - val)
        if best is None or d < best[0] or (d == best[0] and code % 2 == 0):
            best = (d, code)
    return best[1]


def test_round_e4m3_brute_force_exact():
    vals = [Fraction(orc.lib().orc_decode_e4m3(c)) for c in range(0x7F)]
    codes = list(range(0x7F))
    rng = _rng(3)
    samples = list(rng.uniform(0, 448, 3000)) + list(rng.uniform(0, 2.0 ** -5, 2000))
    # every midpoint between neighbours, and just above / below it
    for a, b in zip(vals[:-1], vals[1:]):
        m = (a + b) / 2
        samples += [float(m), math.nextafter(float(m), 0), math.nextafter(float(m), 1000)]
    for s in samples:
        exp = _nearest_exact(Fraction(s), vals, codes)
        assert orc.lib().orc_round_e4m3(s) == exp, s
        assert orc.lib().orc_round_e4m3(-s) == (exp | 0x80), -s


def test_round_e4m3_matches_torch_in_range():
    rng = _rng(4)
    v = np.concatenate([rng.uniform(-448, 448, 200_000),
                        rng.standard_normal(200_000) * 2.0 ** rng.integers(-12, 8, 200_000)])
    v = np.clip(v, -448, 448).astype(np.float32)
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = orc.round_e4m3(v.astype(np.float64))
    assert np.array_equal(got, ref)


@pytest.mark.parametrize("value, code", [
    (448.0, 0x7E), (464.0 - 1e-9, 0x7E), (416.0, 0x7D), (432.0, 0x7E),  # tie 416|448 -> even 0x7E
    (2.0 ** -9, 0x01), (2.0 ** -10, 0x00), (3 * 2.0 ** -10, 0x02), (2.0 ** -6, 0x08),
    (1.0, 0x38), (1.0625, 0x38), (1.1875, 0x3A), (-(2.0 ** -11), 0x80), (-0.0, 0x80),
    (0.0, 0x00), (240.0, 0x77), (256.0, 0x78),
])
def test_round_e4m3_closed_values(value, code):
    # OCP e4m3fn: bias 7, 3 mantissa bits, max 1.75*2^8 = 448, subnormals k*2^-9
    assert orc.lib().orc_round_e4m3(value) == code


# ------------------------------------------------------------------- E8M0
def _floor_log2(a: float) -> int:
    m, e = math.frexp(a)  # a = m * 2^e, m in [0.5, 1)
    return e - 1


def test_e8m0_closed_form_all_bf16_amax():
    c = np.arange(1, 0x7F80, dtype=np.uint16)  # every positive finite bf16
    a = torch.from_numpy(c.view(np.int16)).view(torch.bfloat16).float().numpy()
    got = orc.e8m0_byte(a)
    exp = np.array([max(_floor_log2(float(x)) - 8 + 127, 0) for x in a], dtype=np.int64)
    assert np.array_equal(got.astype(np.int64), exp)
    assert orc.lib().orc_e8m0_byte(0.0) == 0


def test_e8m0_brute_force_smallest_scale():
    """The byte is the smallest b whose scale 2^(b-127) brings amax below
    512 = 2 * (largest e4m3 binade 2^8), i.e. amax/X lands in [256, 512)."""
    rng = _rng(5)
    amax = np.concatenate([(rng.standard_normal(3000) ** 2) * 2.0 ** rng.integers(-100, 100, 3000),
                           2.0 ** np.arange(-118, 120, dtype=np.float64)]).astype(np.float32)
    for a in amax:
        a = float(a)
        if a <= 0:
            continue
        b = next(b for b in range(0, 255) if Fraction(a) / Fraction(2) ** (b - 127) < 512)
        assert orc.lib().orc_e8m0_byte(a) == b, a
        if b > 0:
            assert 256 <= Fraction(a) / Fraction(2) ** (b - 127) < 512


def test_mx_quant_every_bf16_value_under_every_block_exponent():
    """The MXFP8 block quantiser over every finite bf16 value u under every
    block exponent that admits it.  A block's amax is the largest bf16 of
    fp32 exponent field E (E = 1..254), so every u of exponent field <= E
    fits under it; the scale byte must be max(E - 8, 0) and each code
    e4m3(clamp(u 2^(127-b), +-448)), checked against torch's float8_e4m3fn
    cast of the exactly scaled value (fp64 scaling is exact; the result is
    exact in fp32 wherever it can reach an e4m3 rounding boundary)."""
    c = np.arange(1 << 16, dtype=np.uint32)
    fin = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    field = (fin.astype(np.uint32) >> 7) & 0xFF
    rows, bytes_exp = [], []
    for E in range(1, 255):
        vals = fin[field <= E]
        amax = np.uint16((E << 7) | 0x7F)
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blk = np.concatenate([np.full((n, 1), amax, np.uint16), pad.reshape(n, 31)], axis=1)
        rows.append(blk)
        bytes_exp.append(np.full(n, max(E - 8, 0), np.uint8))
    x = np.concatenate(rows)
    want_b = np.concatenate(bytes_exp)
    codes, scales = orc.quant(x, orc.BF16, orc.MXFP8, threads=8)
    assert np.array_equal(scales[:, 0], want_b)
    u = torch.from_numpy(x.view(np.int16)).view(torch.bfloat16).double().numpy()
    v = np.clip(np.ldexp(u, (127 - want_b.astype(np.int64))[:, None]), -448.0, 448.0)
    ref = torch.from_numpy(v.astype(np.float32)).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    bad = np.argwhere(codes != ref)
    assert bad.size == 0, (bad[:5].tolist(), x[tuple(bad[0])] if bad.size else None)
