"""Pins of the oracle's clamped SwiGLU + MXFP8 (the swiglu_oai activation of
vLLM pull request 65478's benchmark script, alpha = 1.702, beta = 1.0,
limit = 7.0).

What ties it to something other than itself:
  - every finite bf16 gate: fl32(glu) equals the fp32 rounding of the
    60-digit decimal value of min(g, limit) * logistic(alpha * min(g, limit));
  - the fp32 activation on random and special (gate, up) pairs equals exact
    rational roundings of the decimal value (clamps, beta, both roundings);
  - whole rows against the brute-force MX quantiser of that activation;
  - alpha = 1, beta = 0, limit = +inf reduces it, bit for bit, to the SiLU
    path, whose own pins are in test_oracle_silu_quant.py;
  - clamping: gates above the limit and ups beyond +-limit act as the limit,
    gates below -limit are not clamped.
"""
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from activation_fp8_quant_amd import inputs
from tests import brute
from tests._compare import ord8

ALPHA, BETA, LIMIT = 1.702, 1.0, 7.0


def _f32(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def _dec(f: Fraction) -> Decimal:
    return Decimal(f.numerator) / Decimal(f.denominator)


def _glu_exact(g: Fraction, alpha=ALPHA, limit=LIMIT) -> Decimal:
    """min(g, limit) * logistic(alpha * min(g, limit)), 60 digits; alpha and
    limit as their fp32 values."""
    lim = _f32(limit) if np.isfinite(limit) else None
    gc = g if lim is None or g < lim else lim
    z = _dec(_f32(alpha) * gc)
    gd = _dec(gc)
    if z < 0:  # gc e^z / (1 + e^z): no overflow for very negative z
        e = z.exp()
        return gd * e / (1 + e)
    return gd / (1 + (-z).exp())


def _act_exact(gb, ub, alpha=ALPHA, beta=BETA, limit=LIMIT) -> Fraction:
    """fl32(fl32(glu) * fl32(clamp(u, +-limit) + beta)) by exact roundings."""
    g = brute.frac_of_bits16(gb, "bf16")
    u = brute.frac_of_bits16(ub, "bf16")
    lim = _f32(limit)
    uc = max(min(u, lim), -lim)
    glu32 = brute.rn_f32(_glu_exact(g, alpha, limit))
    lin32 = brute.rn_f32(uc + _f32(beta))
    return brute.rn_f32(glu32 * lin32)


def _all_finite_bf16():
    c = np.arange(1 << 16, dtype=np.uint32)
    return c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)


@pytest.mark.slow
def test_glu32_every_bf16_gate():
    """fl32(glu) for all 65,280 finite bf16 gates equals the fp32 rounding of
    the 60-digit value (the gate factor the quantiser path uses)."""
    gates = _all_finite_bf16()
    gvals = inputs.bits_to_float(gates).astype(np.float64)
    got = orc.swiglu_glu32(gvals, ALPHA, LIMIT)
    bad = []
    for i in range(gates.size):
        if gates[i] == 0x8000:  # -0 * logistic(0) = -0
            ok = got[i] == 0 and np.signbit(got[i])
        else:
            want = brute.rn_f32(_glu_exact(brute.frac_of_bits16(gates[i], "bf16")))
            ok = Fraction(float(got[i])) == want
        if not ok:
            bad.append((hex(int(gates[i])), float(got[i])))
    assert not bad, bad[:10]


def test_act32_pairs_brute_force():
    """The fp32 activation on random bf16 pairs (the pages' randn * 8 inputs)
    and on pairs that exercise each clamp, beta cancelling up, tiny gates and
    very negative gates."""
    rng = np.random.default_rng(31)
    g = rng.standard_normal(512) * 8.0
    u = rng.standard_normal(512) * 8.0
    special = [(-7.0, -1.0), (7.0, 7.0), (7.5, 7.5), (1e4, -1e4), (-1e4, 3.0), (-60.0, 5.0),
               (-88.0, 7.0), (1e-30, 2.0), (-1e-30, -2.0), (0.0, -1.0), (2.0 ** -130, 1.0),
               (0.25, 2.0 ** -20), (-0.25, -(2.0 ** -30)), (6.9999, 6.9999), (-6.0, -7.5)]
    for k, (a, b) in enumerate(special):
        g[k], u[k] = a, b
    gb, ub = inputs.to_bits(g), inputs.to_bits(u)
    got = orc.swiglu_act32(inputs.bits_to_float(gb).astype(np.float64),
                           inputs.bits_to_float(ub).astype(np.float64), ALPHA, BETA, LIMIT)
    for j in range(g.size):
        want = _act_exact(gb[j], ub[j])
        assert Fraction(float(got[j])) == want, (j, float(g[j]), float(u[j]), float(got[j]))


def _mx_row_brute(gbits, ubits, qin=orc.QIN_DEFAULT):
    a = [_act_exact(gb, ub) for gb, ub in zip(gbits, ubits)]
    if qin == orc.QIN_BF16:
        a = [brute.frac_of_bits16(brute.round16(v, "bf16")[0], "bf16") for v in a]
    codes, scales = [], []
    for k in range(0, len(a), 32):
        q, s = brute.quant_mx(a[k:k + 32])
        codes += q
        scales.append(s)
    return codes, scales


@pytest.mark.parametrize("qin", [orc.QIN_DEFAULT, orc.QIN_BF16])
def test_swiglu_mx_rows_brute_force(qin):
    """Whole rows (randn * 8, as the pages' benchmark draws them) against the
    exact activation and the brute-force MX quantiser; the bf16 copy is the
    rounding of the exact fp32 activation."""
    I = 128
    gu = inputs.gate_up_inputs(2, I, seed=32, std=8.0)
    out = orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, qin=qin)
    for i in range(2):
        codes, scales = _mx_row_brute(gu[i, :I], gu[i, I:], qin)
        assert np.array_equal(ord8(out["values"][i]), ord8(np.array(codes, np.uint8)))
        assert list(out["scales"][i]) == scales
        for j in range(I):
            c, _ = brute.round16(_act_exact(gu[i, j], gu[i, I + j]), "bf16")
            assert (c & 0x7FFF) == (int(out["act"][i, j]) & 0x7FFF), (i, j)


def test_reduces_to_silu():
    """alpha = 1, beta = 0, limit = +inf is SiLU-and-mul: codes, scales and
    copy equal the SiLU path's bit for bit (inputs with extreme gates)."""
    gu = inputs.gate_up_inputs(16, 256, seed=33, std=4.0)
    ext = inputs.to_bits(np.array([-95.0, -88.5, -200.0, 100.0, 1e30, -1e30, 0.0, -0.0]))
    gu[0, :8] = ext
    for qin in (orc.QIN_DEFAULT, orc.QIN_BF16):
        a = orc.swiglu_oai_quant(gu, 1.0, 0.0, float("inf"), qin=qin)
        b = orc.silu_quant(gu, orc.MXFP8, qin=qin)
        for k in ("values", "scales", "act"):
            assert np.array_equal(a[k], b[k]), (qin, k)


def test_clamps():
    """Gates above the limit act as the limit and gates below -limit are not
    clamped; ups beyond +-limit act as +-limit."""
    rng = np.random.default_rng(34)
    M, I = 4, 256
    g = rng.standard_normal((M, I)) * 3.0
    u = rng.standard_normal((M, I)) * 3.0
    hi_g = rng.uniform(7.0, 40.0, size=(M, I)) * (rng.random((M, I)) < 0.3)
    g_cl = np.where(hi_g > 0, LIMIT, g)
    g_big = np.where(hi_g > 0, hi_g, g)
    big_u = rng.uniform(7.0, 40.0, size=(M, I)) * np.sign(rng.standard_normal((M, I)))
    mask_u = rng.random((M, I)) < 0.3
    u_cl = np.where(mask_u, np.sign(big_u) * LIMIT, u)
    u_big = np.where(mask_u, big_u, u)
    a = orc.swiglu_oai_quant(np.concatenate([inputs.to_bits(g_big), inputs.to_bits(u_big)], 1),
                             ALPHA, BETA, LIMIT)
    b = orc.swiglu_oai_quant(np.concatenate([inputs.to_bits(g_cl), inputs.to_bits(u_cl)], 1),
                             ALPHA, BETA, LIMIT)
    for k in ("values", "scales", "act"):
        assert np.array_equal(a[k], b[k]), k
    # below -limit the gate is not clamped: glu(-20) is about -20 e^-34, far
    # from glu(-7)
    low = orc.swiglu_glu32(np.array([-20.0, -7.0]), ALPHA, LIMIT)
    assert abs(low[0]) < 1e-13 and abs(low[1]) > 4e-5


def test_mx_only():
    gu = inputs.gate_up_inputs(1, 128, seed=1, std=1.0)
    for mode in (orc.BLOCK128, orc.PER_TOKEN):
        with pytest.raises(ValueError):
            orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, mode)
