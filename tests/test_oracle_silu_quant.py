"""Pins of the oracle's SiLU-and-mul and standalone quantisers: exhaustive
SiLU rounding against 60-digit decimal arithmetic, exact brute force on tiny
rows, and the quantiser invariants (dequantise-then-compare, saturation,
monotonicity, scale closed forms, cross-mode identities)."""
from decimal import Decimal
from fractions import Fraction

import numpy as np
import pytest

import oracle as orc
from activation_fp8_quant_amd import inputs
from tests import brute
from tests._compare import ord8


def _all_finite_bf16():
    c = np.arange(1 << 16, dtype=np.uint32)
    return c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)


def _silu_exact(g: Fraction) -> Decimal:
    gd = Decimal(g.numerator) / Decimal(g.denominator)
    if gd < 0:  # g e^g / (1 + e^g): no overflow for very negative g
        e = gd.exp()
        return gd * e / (1 + e)
    return gd / (1 + (-gd).exp())


@pytest.mark.slow
def test_silu_bf16_rounding_exhaustive():
    """bf16(silu(g)) for every finite bf16 gate equals the rounding of the
    60-digit value.  Read through the 1x128 SiLU-and-mul with up = 1, whose
    activation copy is bf16(bf16(silu(g)) * 1)."""
    gates = _all_finite_bf16()
    n = gates.size
    pad = (-n) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)])
    one = inputs.to_bits(np.ones(1))[0]
    rows = g.reshape(-1, 128)
    gu = np.concatenate([rows, np.full_like(rows, one)], axis=1)
    out = orc.silu_quant(gu, orc.BLOCK128, threads=8)
    act = out["act"].ravel()[:n]
    bad = []
    for i in range(n):
        gf = brute.frac_of_bits16(gates[i], "bf16")
        code, _ = brute.round16(_silu_exact(gf), "bf16")
        if gates[i] == 0x8000:
            code = 0x8000  # silu(-0) = -0 * logistic(0) = -0 (IEEE sign of zero)
        if code != int(act[i]):
            bad.append((int(gates[i]), code, int(act[i])))
    assert not bad, bad[:10]


def _silu_fp32_act(gb, ub):
    """fl32(fl32(silu(g)) * u) from 60-digit silu and exact roundings (the
    fp32 SiLU-and-mul of the MXFP8 path)."""
    gf = brute.frac_of_bits16(gb, "bf16")
    uf = brute.frac_of_bits16(ub, "bf16")
    a = brute.rn_f32(brute.rn_f32(_silu_exact(gf)) * uf)
    if a == 0:  # a zero keeps the IEEE sign of the product (silu(g) has the sign of g)
        return Decimal("-0") if ((int(gb) ^ int(ub)) >> 15) & 1 else Decimal(0)
    return a


def test_silu_fp32_product_brute_force():
    """MXFP8 activation: fl32(fl32(silu(g)) * u), checked with decimal silu
    and exact roundings on random bf16 pairs (incl. large |g|), and on gates
    whose silu is an fp32 subnormal or zero times large up values, where
    rounding silu to fp32 first decides the result."""
    rng = np.random.default_rng(21)
    I = 256
    g = rng.standard_normal(I) * 4.0
    g[:8] = [-95.0, -88.5, -60.0, -20.0, 20.0, 60.0, 0.0, -1e-30]
    u = rng.standard_normal(I) * 2.0
    g[8:16] = [-95.0, -100.0, -103.0, -109.0, -118.0, -90.0, -87.5, -150.0]
    u[8:16] = [1e30, -(2.0 ** 40), 1e30, 1e30, 1e30, 2.0 ** 100, 2.0 ** 60, 1e38]
    gu = np.concatenate([inputs.to_bits(g), inputs.to_bits(u)])[None, :]
    out = orc.silu_quant(gu, orc.MXFP8)
    act = out["act"][0]
    for j in range(I):
        c, _ = brute.round16(_silu_fp32_act(gu[0, j], gu[0, I + j]), "bf16")
        assert c == int(act[j]), j
    # fl32(silu(-109)) is -0, so the product is -0 whatever up is
    assert int(act[11]) == 0x8000


def _silu_mx_row_brute(gbits, ubits):
    """Exact activation of one row then the MX quantiser of the brute force."""
    a = [_silu_fp32_act(gb, ub) for gb, ub in zip(gbits, ubits)]
    codes, scales = [], []
    for k in range(0, len(a), 32):
        q, s = brute.quant_mx(a[k:k + 32])
        codes += q
        scales.append(s)
    return codes, scales


def _silu_b128_row_brute(gbits, ubits):
    a = []
    for gb, ub in zip(gbits, ubits):
        gf = brute.frac_of_bits16(gb, "bf16")
        uf = brute.frac_of_bits16(ub, "bf16")
        _, sg = brute.round16(_silu_exact(gf), "bf16")
        _, av = brute.round16(sg * uf, "bf16")
        a.append(av)
    codes, scales = [], []
    for k in range(0, len(a), 128):
        q, s = brute.quant_fp32scale(a[k:k + 128])
        codes += q
        scales.append(s)
    return codes, scales


@pytest.mark.parametrize("mode", [orc.MXFP8, orc.BLOCK128])
def test_silu_quant_matches_brute_force(mode):
    I = 256
    gu = inputs.gate_up_inputs(2, I, seed=22, std=2.0)
    out = orc.silu_quant(gu, mode)
    for i in range(2):
        fn = _silu_mx_row_brute if mode == orc.MXFP8 else _silu_b128_row_brute
        codes, scales = fn(gu[i, :I], gu[i, I:])
        assert np.array_equal(ord8(out["values"][i]), ord8(np.array(codes, np.uint8)))
        if mode == orc.MXFP8:
            assert list(out["scales"][i]) == scales
        else:
            assert np.array_equal(out["scales"][i], np.array(scales, np.float32))


def test_silu_mx_bf16_first_matches_brute_force():
    """The bf16-first MXFP8 variant quantises RNE_bf16(fl32(fl32(silu(g)) u)),
    the activation as the unfused chain stores it (decimal silu, exact
    roundings, brute-force MX quantiser)."""
    I = 256
    gu = inputs.gate_up_inputs(2, I, seed=23, std=2.0)
    out = orc.silu_quant(gu, orc.MXFP8, qin=orc.QIN_BF16)
    for i in range(2):
        a = []
        for gb, ub in zip(gu[i, :I], gu[i, I:]):
            _, ab = brute.round16(_silu_fp32_act(gb, ub), "bf16")
            a.append(ab)
        codes, scales = [], []
        for k in range(0, I, 32):
            q, s = brute.quant_mx(a[k:k + 32])
            codes += q
            scales.append(s)
        assert np.array_equal(ord8(out["values"][i]), ord8(np.array(codes, np.uint8)))
        assert list(out["scales"][i]) == scales
    # the optional bf16 copy is the same in both variants
    assert np.array_equal(out["act"], orc.silu_quant(gu, orc.MXFP8)["act"])


def test_silu_per_token_rejected():
    gu = inputs.gate_up_inputs(1, 128, seed=1, std=1.0)
    with pytest.raises(ValueError):
        orc.silu_quant(gu, orc.PER_TOKEN)


# --------------------------------------------------------------- quantiser
def _e4m3_spacing(v):
    """Spacing of e4m3fn values around magnitude v (<= 448)."""
    a = np.abs(v)
    e = np.floor(np.log2(np.maximum(a, 2.0 ** -6)))
    return 2.0 ** (e - 3)


@pytest.mark.parametrize("in_dtype", [orc.BF16, orc.FP32])
@pytest.mark.parametrize("mode", [orc.MXFP8, orc.BLOCK128, orc.PER_TOKEN])
def test_dequantise_then_compare(mode, in_dtype):
    """|v - val(q)| <= half the local e4m3 spacing (plus the fp32 quotient's
    rounding) for in-range v; saturated codes for |v| > 448; monotone codes."""
    rng = np.random.default_rng(23)
    M, n = 16, 512
    x = rng.standard_normal((M, n)) * 2.0 ** rng.integers(-10, 10, (M, 1))
    x[0, :] = rng.standard_normal(n) * 1e-38      # fp32-subnormal-ish block
    x[1, ::7] *= 300.0                            # dominated blocks
    if in_dtype == orc.BF16:
        xb = inputs.to_bits(x)
        v_in = inputs.bits_to_float(xb).astype(np.float64)
    else:
        xb = x.astype(np.float32)
        v_in = xb.astype(np.float64)
    q, s = orc.quant(xb, in_dtype, mode)
    deq = orc.decode_e4m3(q)
    G = 32 if mode == orc.MXFP8 else 128 if mode == orc.BLOCK128 else n
    for i in range(M):
        for k in range(0, n, G):
            blk = v_in[i, k:k + G]
            if mode == orc.MXFP8:
                X = 2.0 ** (int(s[i, k // 32]) - 127)
                v = blk / X
                tol = 0.0
            else:
                sc = float(s[i, k // G] if mode == orc.BLOCK128 else s[i, 0])
                if sc == 0.0:
                    assert not (q[i, k:k + G] & 0x7F).any()
                    continue
                v = (blk.astype(np.float32) / np.float32(sc)).astype(np.float64)
                tol = 0.0
            dq = deq[i, k:k + G]
            inr = np.abs(v) <= 448
            err = np.abs(v[inr] - dq[inr])
            assert np.all(err <= _e4m3_spacing(v[inr]) / 2 + tol)
            assert np.all(np.abs(dq[~inr]) == 448)
            order = np.argsort(blk, kind="stable")
            assert np.all(np.diff(dq[order]) >= 0)


def test_fp32_scale_closed_form_max_element():
    """s * 448 reproduces the group amax within fp32 rounding, and the
    largest element quantises to +-448 (code 0x7E / 0xFE)."""
    rng = np.random.default_rng(24)
    x = inputs.to_bits(rng.standard_normal((8, 1024)) * 5.0)
    v = inputs.bits_to_float(x).astype(np.float64)
    for mode, G in ((orc.BLOCK128, 128), (orc.PER_TOKEN, 1024)):
        q, s = orc.quant(x, orc.BF16, mode)
        for i in range(8):
            for k in range(0, 1024, G):
                blk = v[i, k:k + G]
                A = np.abs(blk).max()
                sc = float(s[i, k // G])
                assert abs(sc * 448 - A) <= A * 2.0 ** -23
                j = np.argmax(np.abs(blk))
                assert q[i, k + j] & 0x7F == 0x7E


def test_mx_scale_puts_block_max_in_top_binade():
    rng = np.random.default_rng(25)
    x = inputs.to_bits(rng.standard_normal((8, 1024)) * 2.0 ** rng.integers(-30, 30, (8, 1)))
    v = inputs.bits_to_float(x).astype(np.float64)
    q, s = orc.quant(x, orc.BF16, orc.MXFP8)
    for i in range(8):
        for k in range(32):
            A = np.abs(v[i, 32 * k:32 * k + 32]).max()
            r = A / 2.0 ** (int(s[i, k]) - 127)
            assert 256 <= r < 512


def test_per_token_equals_block128_at_width_128():
    rng = np.random.default_rng(26)
    x = inputs.to_bits(rng.standard_normal((32, 128)) * 3.0)
    a = orc.quant(x, orc.BF16, orc.PER_TOKEN)
    b = orc.quant(x, orc.BF16, orc.BLOCK128)
    assert np.array_equal(a[0], b[0]) and np.array_equal(a[1], b[1])


def test_group_permutation_equivariance():
    rng = np.random.default_rng(27)
    x = inputs.to_bits(rng.standard_normal((4, 256)) * 3.0)
    perm = np.concatenate([rng.permutation(32) + 32 * k for k in range(8)])
    for mode in (orc.MXFP8, orc.BLOCK128):
        if mode == orc.BLOCK128:
            perm = np.concatenate([rng.permutation(128) + 128 * k for k in range(2)])
        q, s = orc.quant(x, orc.BF16, mode)
        qp, sp = orc.quant(x[:, perm], orc.BF16, mode)
        assert np.array_equal(qp, q[:, perm]) and np.array_equal(sp, s)


def test_quant_rows_brute_force_fp32_input():
    rng = np.random.default_rng(28)
    x = (rng.standard_normal((2, 256)) * 2.0 ** rng.integers(-20, 20, (2, 256))).astype(np.float32)
    for mode, G in ((orc.MXFP8, 32), (orc.BLOCK128, 128), (orc.PER_TOKEN, 256)):
        q, s = orc.quant(x, orc.FP32, mode)
        for i in range(2):
            for k in range(0, 256, G):
                u = [Fraction(float(t)) for t in x[i, k:k + G]]
                if mode == orc.MXFP8:
                    codes, b = brute.quant_mx(u)
                    assert int(s[i, k // 32]) == b
                else:
                    codes, sc = brute.quant_fp32scale(u)
                    assert np.float32(s[i, k // G]) == sc
                assert np.array_equal(ord8(q[i, k:k + G]), ord8(np.array(codes, np.uint8)))


def test_fp32_scale_underflow_gives_zero_codes():
    """Reading R25: a 1x128 / per-token group whose amax / 448 underflows
    fp32 (amax at most 224 * 2^-149: the quotient is at most half the least
    subnormal, and the tie goes to the even zero) stores s = 0, and every
    code is 0x00 as for the all-zero group.  The next amax up stores the
    least subnormal, and its codes follow the quotient as usual."""
    tiny = np.float32(2.0 ** -149)
    x = np.zeros((2, 128), np.float32)
    x[0, :] = -tiny
    x[0, 5] = np.float32(224) * tiny
    x[1, :] = tiny
    x[1, 9] = np.float32(225) * tiny
    for mode in (orc.BLOCK128, orc.PER_TOKEN):
        q, s = orc.quant(x, orc.FP32, mode)
        assert s[0, 0] == 0 and not np.any(q[0])
        assert s[1, 0] == tiny
        assert q[1, 9] == 0x76                              # 225 -> 224 = 1.75 * 2^7
        assert np.all(q[1, np.arange(128) != 9] == 0x38)    # quotient 1.0
        # the same through the exact brute force
        for i in range(2):
            codes, sc = brute.quant_fp32scale([Fraction(float(t)) for t in x[i]])
            assert np.float32(s[i, 0]) == sc and list(q[i]) == codes
