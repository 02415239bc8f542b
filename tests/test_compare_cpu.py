"""The parity comparator itself, on the CPU: results built from the oracle
with a planted one-value rounding flip of a group's largest activation (the
reading R14 case) pass, with the group listed; planted mistakes that the
contract does not allow -- a scale two fp32 ulps off, a code two steps off,
an E8M0 step without a flip behind it, more inexact groups than 0.1 % --
fail."""
import numpy as np
import pytest

import oracle as orc
from activation_fp8_quant_amd import inputs
from tests._compare import check_quant, check_scales


def _case(mode, dtype="bf16", M=1024, H=1024, seed=0):
    rng = np.random.default_rng(seed)
    u = inputs.to_bits(rng.standard_normal((M, H)) * 2.0 ** rng.integers(-4, 4, (M, 1)), dtype)
    q, s = orc.quant(u, orc.BF16 if dtype == "bf16" else orc.FP16, mode)
    return u, q, s


def _flip_max(u, row, lo, hi, up):
    """The row's group [lo, hi) with its largest magnitude moved one value."""
    v = u.copy()
    g = v[row, lo:hi]
    mag = g & 0x7FFF
    a = int(mag.max())
    sel = mag == a
    g[sel] = (g[sel] & 0x8000) | np.uint16(a + (1 if up else -1))
    return v


@pytest.mark.parametrize("mode,width", [(orc.BLOCK128, 128), (orc.PER_TOKEN, 1024)])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_r14_flip_is_explained_and_listed(mode, width, dtype):
    u, q, s = _case(mode, dtype)
    fam = orc.BF16 if dtype == "bf16" else orc.FP16
    for up in (True, False):
        v = _flip_max(u, 3, 0, width, up)
        gq, gs = orc.quant(v, fam, mode)
        assert not np.array_equal(gs, s)
        n1, nbad, listed = check_quant(gq, gs, q, s, mode, "flip", u=u, dtype=dtype)
        assert nbad == 1 and listed[0][1].startswith("R14") and listed[0][0] == 3 * (1024 // width)
        assert n1 <= 1024 * 1024 // 1000


def test_mx_power_of_two_flip_is_explained():
    """An MXFP8 block whose largest value sits just below a power of two:
    moved one bf16 value up, its E8M0 byte steps and every code of the block
    moves (up to 8 steps); the comparator recognises the flip."""
    u, q, s = _case(orc.MXFP8)
    one_below = inputs.to_bits(np.array([1.0 - 2.0 ** -8]))[0]
    u[5, :32] = inputs.to_bits(np.random.default_rng(1).uniform(-0.9, 0.9, 32))
    u[5, 7] = one_below
    q, s = orc.quant(u, orc.BF16, orc.MXFP8)
    v = _flip_max(u, 5, 0, 32, True)
    gq, gs = orc.quant(v, orc.BF16, orc.MXFP8)
    assert int(gs[5, 0]) == int(s[5, 0]) + 1
    n1, nbad, listed = check_quant(gq, gs, q, s, orc.MXFP8, "mx-flip", u=u, dtype="bf16")
    assert nbad == 1


def test_unexplained_differences_fail():
    u, q, s = _case(orc.BLOCK128)
    # a scale two fp32 ulps off
    gs = s.copy()
    gs.view(np.uint32)[2, 1] += 2
    with pytest.raises(AssertionError):
        check_scales(gs, s, orc.BLOCK128, "two-ulp", u=u, dtype="bf16")
    # a code two steps off
    gq = q.copy()
    gq[1, 10] = (gq[1, 10] & 0x80) | ((gq[1, 10] & 0x7F) + 2 if (gq[1, 10] & 0x7F) < 0x7C else (gq[1, 10] & 0x7F) - 2)
    with pytest.raises(AssertionError):
        check_quant(gq, s, q, s, orc.BLOCK128, "two-steps", u=u, dtype="bf16")
    # an E8M0 step with no flip behind it
    u2, q2, s2 = _case(orc.MXFP8)
    gs2 = s2.copy()
    gs2[0, 0] += 1
    with pytest.raises(AssertionError):
        check_quant(q2, gs2, q2, s2, orc.MXFP8, "bare-step", u=u2, dtype="bf16")
    # an R14 group among 512 groups (budget 0)
    u, q, s = _case(orc.BLOCK128, M=64)
    v = _flip_max(u, 0, 0, 128, True)
    gq, gs = orc.quant(v, orc.BF16, orc.BLOCK128)
    with pytest.raises(AssertionError):
        check_quant(gq, gs, q, s, orc.BLOCK128, "too-many", u=u, dtype="bf16")


def _minus_one(q, idx):
    """q with the codes at flat indices idx moved one step toward zero."""
    g = q.copy().ravel()
    for i in idx:
        g[i] = (g[i] & 0x80) | ((g[i] & 0x7F) - 1)
    return g.reshape(q.shape)


def test_one_apart_codes_are_budgeted():
    u, q, s = _case(orc.PER_TOKEN, M=2, H=1024)        # 2048 codes: budget 2
    idx = np.flatnonzero((q.ravel() & 0x7F) > 8)[:3]
    check_quant(_minus_one(q, idx[:2]), s, q, s, orc.PER_TOKEN, "two", u=u, dtype="bf16")
    with pytest.raises(AssertionError):
        check_quant(_minus_one(q, idx), s, q, s, orc.PER_TOKEN, "three", u=u, dtype="bf16")
