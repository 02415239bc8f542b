"""The gfx950 instructions and fast arithmetic the kernels rely on, checked
on the GPU over exhaustive input sets (the probe library in tests/probe
applies the library's own device primitives element-wise):

  * the fp32 scale amax/448 of the 1x128 and per-token quantisers: on the
    fast path (amax >= 2^-83) a product with RN(1/448) plus one correction,
    and RN(1/s) as the hardware reciprocal plus one Newton step.  Both must
    equal the IEEE divisions (numpy float32 on the host) for every fp32
    mantissa at every exponent of the fast path (and, as probed, from
    2^-116 up); below 2^-83 the kernels take the IEEE division;
  * the quotient u/s a quantiser forms, for u = +-amax (quotients at 448 and
    at most one ulp beyond it) and random u, every amax mantissa at boundary
    and middle exponents: correctly rounded (the fast path's Markstein
    correction, or the IEEE division below 2^-83) wherever it can decide an
    e4m3 code (|u/s| >= 2^-11; smaller quotients round to a zero code);
  * v_cvt_pk_fp8_f32, unclamped, on every fp32 in [448, 464] of either sign
    (what the fast path can hand it beyond 448 is at most 448(1 + 2^-23))
    and on every fp32 in [2^-10, 464) of either sign, against the oracle's
    e4m3 rounding;
  * v_cvt_pk_bf16_f32 on every bf16 neighbourhood of the fp32 line: each of
    the 2^16 upper halves with the lower halves that decide round to nearest
    even (0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF and two random), against the
    oracle's bf16 rounding;
  * the fp32-direct norm's inverse RMS fl32(1 / sqrt(ss / cols + eps)) (its
    fast path and the fallback to the fp64 formula) against the formula in
    numpy float64, on random sums and on sums whose result sits on an fp32
    rounding midpoint.
"""
import concurrent.futures
import ctypes
import os

import numpy as np
import pytest
import torch

import oracle as orc
from tests._gpu import HOST_THREADS

pytestmark = pytest.mark.gpu

PROBE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "probe", "libafq_probe.so")


def _probe():
    if not os.path.exists(PROBE):
        raise FileNotFoundError(f"{PROBE} is missing: build it with `python -m tests.probe.build`")
    L = ctypes.CDLL(PROBE)
    P, I64 = ctypes.c_void_p, ctypes.c_int64
    L.afqp_scale.argtypes = [P, P, P, P, I64, P]
    L.afqp_quotient.argtypes = [P, P, P, I64, P]
    L.afqp_cvt8_e4m3.argtypes = [P, P, I64, P]
    L.afqp_e4m3_range.argtypes = [ctypes.c_uint32, P, I64, P]
    L.afqp_pack_bf16.argtypes = [P, P, I64, P]
    L.afqp_inv_rms.argtypes = [P, ctypes.c_int32, ctypes.c_float, P, P, I64, P]
    L.afqp_issue.argtypes = [ctypes.c_int, P, I64, ctypes.c_int32, P]
    L.afqp_rows_pattern.argtypes = [P, I64, P, P, P, P, I64, ctypes.c_int32, ctypes.c_int32, P]
    for f in (L.afqp_scale, L.afqp_quotient, L.afqp_cvt8_e4m3, L.afqp_e4m3_range, L.afqp_pack_bf16,
              L.afqp_inv_rms, L.afqp_issue, L.afqp_rows_pattern):
        f.restype = ctypes.c_int
    return L


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _binade(E: int) -> np.ndarray:
    """Every fp32 of exponent field E, ascending, as float32."""
    return ((np.uint32(E) << np.uint32(23)) | np.arange(1 << 23, dtype=np.uint32)).view(np.float32)


def _gpu_scale(L, a: np.ndarray):
    at = torch.from_numpy(a).cuda()
    s, r = torch.empty_like(at), torch.empty_like(at)
    f = torch.empty(a.size, dtype=torch.uint8, device="cuda")
    rc = L.afqp_scale(at.data_ptr(), s.data_ptr(), r.data_ptr(), f.data_ptr(), a.size, _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return s.cpu().numpy(), r.cpu().numpy(), f.cpu().numpy().astype(bool)


FAST_MIN = np.float32(2.0 ** -83)


def test_fp32_scale_and_reciprocal_every_mantissa_every_exponent():
    """s = amax/448 and 1/s against IEEE float32 division for all 2^23
    mantissas of every exponent field 0..254 (2.1 G amax values): s
    bit-exact everywhere, the fast flag set exactly for amax >= 2^-83, 1/s
    bit-exact wherever the quantiser uses it (the fast flag)."""
    L = _probe()
    four48, one = np.float32(448.0), np.float32(1.0)
    fast_seen = 0
    for E0 in range(0, 255, 8):
        Es = list(range(E0, min(E0 + 8, 255)))
        print(f"case fp32 scale exponent fields {Es[0]}..{Es[-1]}", flush=True)
        a = np.concatenate([_binade(E) for E in Es])
        s, r, fast = _gpu_scale(L, a)
        with np.errstate(divide="ignore", over="ignore"):
            s_ref = a / four48
            r_ref = one / s_ref
        bad = np.flatnonzero(s.view(np.uint32) != s_ref.view(np.uint32))
        assert bad.size == 0, [(float(a[i]), float(s[i]), float(s_ref[i])) for i in bad[:5]]
        fast_ref = a >= FAST_MIN
        assert np.array_equal(fast, fast_ref), np.flatnonzero(fast != fast_ref)[:5]
        bad = np.flatnonzero(fast & (r.view(np.uint32) != r_ref.view(np.uint32)))
        assert bad.size == 0, [(float(a[i]), float(r[i]), float(r_ref[i])) for i in bad[:5]]
        fast_seen += int(fast.sum())
    assert fast_seen > 0


@pytest.mark.parametrize("E", [1, 11, 12, 20, 43, 44, 45, 50, 100, 127, 128, 200, 253, 254])
def test_fp32_quotient_correctly_rounded(E):
    """The quantiser's quotient u/s for every amax mantissa of exponent field
    E (fields 44 up, amax >= 2^-83: the fast path; below it the IEEE
    division), with u = amax, -amax (quotients at 448 or one ulp beside it)
    and a random |u| <= amax: bit-exact against IEEE float32 division
    wherever |u/s| >= 2^-11, and below that both under 2^-10 with the same
    sign (a zero code either way); some quotients land in
    (448, 448(1 + 2^-23)] on the fast path, none beyond."""
    L = _probe()
    a = _binade(E)
    rng = np.random.default_rng(E)
    frac = rng.random(a.size).astype(np.float32)
    u_rand = (a * frac) * np.where(rng.random(a.size) < 0.5, np.float32(-1), np.float32(1))
    u = np.concatenate([a, -a, u_rand.astype(np.float32)])
    aa = np.concatenate([a, a, a])
    ut, at = torch.from_numpy(u).cuda(), torch.from_numpy(aa).cuda()
    q = torch.empty_like(ut)
    rc = L.afqp_quotient(ut.data_ptr(), at.data_ptr(), q.data_ptr(), u.size, _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    q = q.cpu().numpy()
    q_ref = u / (aa / np.float32(448.0))
    big = np.abs(q_ref) >= np.float32(2.0 ** -11)
    bad = np.flatnonzero(big & (q.view(np.uint32) != q_ref.view(np.uint32)))
    assert bad.size == 0, [(float(u[i]), float(aa[i]), float(q[i]), float(q_ref[i])) for i in bad[:5]]
    small = ~big
    assert bool((np.abs(q[small]) < np.float32(2.0 ** -10)).all())
    assert np.array_equal(np.signbit(q[small]), np.signbit(q_ref[small]))
    above = int((np.abs(q_ref) > np.float32(448.0)).sum())
    if a[0] >= FAST_MIN:   # what the unclamped conversion can receive: at most 448(1 + 2^-23)
        assert above > 0 and float(np.abs(q_ref).max()) == float(np.nextafter(np.float32(448), np.float32(512)))
    print(f"[sweep] quotient E={E}: {u.size} quotients, {above} above 448", flush=True)


def _oracle_e4m3(bits: np.ndarray) -> np.ndarray:
    """The oracle's e4m3 rounding of fp32 bit patterns, over host threads."""
    out = np.empty(bits.size, np.uint8)
    chunk = 1 << 22

    def run(i):
        v = bits[i:i + chunk].view(np.float32).astype(np.float64)
        out[i:i + chunk] = orc.round_e4m3(v)

    with concurrent.futures.ThreadPoolExecutor(HOST_THREADS) as ex:
        list(ex.map(run, range(0, bits.size, chunk)))
    return out


def _gpu_e4m3_range(L, base: int, n: int) -> np.ndarray:
    codes = torch.empty(n, dtype=torch.uint8, device="cuda")
    rc = L.afqp_e4m3_range(base, codes.data_ptr(), n, _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    return codes.cpu().numpy()


@pytest.mark.parametrize("sign", [0, 1])
def test_cvt_fp8_unclamped_448_to_464(sign):
    """v_cvt_pk_fp8_f32 without a clamp on every fp32 from just below 448 to
    464 inclusive: every one gives +-448 (0x7E / 0xFE), as the oracle's
    rounding of the clamped value does."""
    L = _probe()
    lo = int(np.float32(448.0).view(np.uint32)) - 7
    hi = int(np.float32(464.0).view(np.uint32))
    n = hi - lo + 1
    assert n % 8 == 0
    base = lo | (sign << 31)
    got = _gpu_e4m3_range(L, base, n)
    bits = np.arange(base, base + n, dtype=np.uint64).astype(np.uint32)
    want = _oracle_e4m3(bits)
    assert bool((want == (0x7E | (sign << 7))).all())
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(int(bits[i])), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("sign", [0, 1])
def test_cvt_fp8_every_fp32_below_464(sign):
    """v_cvt_pk_fp8_f32 on every fp32 in [2^-10, 464) of one sign (exponent
    fields 117..135; smaller magnitudes round to zero, covered by the
    structured test): 159 M values against the oracle's e4m3 rounding."""
    L = _probe()
    top = int(np.float32(464.0).view(np.uint32))
    start = 117 << 23
    step = 1 << 24
    for b0 in range(start, top, step):
        n = min(step, top - b0)
        base = b0 | (sign << 31)
        print(f"case e4m3 sweep base {base:#010x} n {n}", flush=True)
        got = _gpu_e4m3_range(L, base, n)
        bits = np.arange(base, base + n, dtype=np.uint64).astype(np.uint32)
        want = _oracle_e4m3(bits)
        bad = np.flatnonzero(got != want)
        assert bad.size == 0, [(hex(int(bits[i])), hex(got[i]), hex(want[i])) for i in bad[:5]]


def test_cvt_bf16_round_to_nearest_even_classes():
    """v_cvt_pk_bf16_f32 (the kernels' dtype rounding) on every upper half
    of a finite fp32 combined with the lower halves that decide round to
    nearest even -- below, at and above the midpoint, the ends, and two
    random -- against the oracle's bf16 rounding (overflow to infinity
    included)."""
    L = _probe()
    hi = np.arange(1 << 16, dtype=np.uint32)
    hi = hi[((hi >> 7) & 0xFF) != 0xFF]
    rng = np.random.default_rng(5)
    lows = np.array([0, 1, 0x7FFF, 0x8000, 0x8001, 0xFFFF], np.uint32)
    bits = np.concatenate([(hi << 16) | lw for lw in lows]
                          + [(hi << 16) | rng.integers(0, 1 << 16, hi.size).astype(np.uint32)
                             for _ in range(2)])
    v = bits.view(np.float32)
    pad = (-v.size) % 8
    v = np.concatenate([v, np.zeros(pad, np.float32)])
    vt = torch.from_numpy(v).cuda()
    out = torch.empty(v.size, dtype=torch.int16, device="cuda")
    rc = L.afqp_pack_bf16(vt.data_ptr(), out.data_ptr(), v.size, _stream())
    assert rc == 0, rc
    torch.cuda.synchronize()
    got = out.cpu().numpy().view(np.uint16)[:bits.size]
    want = orc.round_bf16(v[:bits.size].astype(np.float64))
    bad = np.flatnonzero(got != want)
    assert bad.size == 0, [(hex(int(bits[i])), hex(got[i]), hex(want[i])) for i in bad[:5]]


@pytest.mark.parametrize("cols,eps", [(4096, 1e-6), (2048, 1e-6), (1536, 1e-6), (512, 1e-6), (6144, 1e-5),
                                      (2176, 0.0), (7168, 1e-6)])
def test_fp32_direct_inverse_rms(cols, eps):
    """The fp32-direct norm's inverse RMS, inv_rms_f32q(ss, cols, eps),
    against fl32(1 / sqrt(ss / cols + eps)) evaluated in numpy float64
    (IEEE division, sum, square root and reciprocal), bit for bit:
      * 2^20 random sums of squares, cols * 10^U(-30, 30): the fast path
        must give at least 99.99 % of them;
      * 2^20 sums whose result lies within about 2^-50 of an fp32 rounding
        midpoint (x = 1 / m^2 for the midpoint m of two fp32 neighbours):
        the fast path must decline almost all of them, so the fallback runs;
      * zero (with eps = 0: infinity), and sums at the ends of the range."""
    L = _probe()
    rng = np.random.default_rng(cols)
    n = 1 << 20
    e64 = np.float64(np.float32(eps))
    ss_rand = cols * 10.0 ** rng.uniform(-30, 30, n)
    f = (2.0 ** rng.uniform(-40, 40, n)).astype(np.float32)
    m = (f.astype(np.float64) + np.nextafter(f, np.float32(np.inf)).astype(np.float64)) / 2
    ss_mid = (1.0 / (m * m) - e64) * cols
    ss_mid = ss_mid[ss_mid > 0]
    special = np.array([0.0, 2.0 ** -1000, 2.0 ** -266, 1.0, float(cols), 2.0 ** 600, 1e300], np.float64)
    print(f"case inverse RMS cols={cols} eps={eps}", flush=True)
    for name, ss in (("random", ss_rand), ("midpoint", ss_mid), ("special", special)):
        st = torch.from_numpy(np.ascontiguousarray(ss)).cuda()
        inv = torch.empty(ss.size, dtype=torch.float32, device="cuda")
        fast = torch.empty(ss.size, dtype=torch.uint8, device="cuda")
        rc = L.afqp_inv_rms(st.data_ptr(), cols, eps, inv.data_ptr(), fast.data_ptr(), ss.size, _stream())
        assert rc == 0, rc
        torch.cuda.synchronize()
        got, fast = inv.cpu().numpy(), fast.cpu().numpy().astype(bool)
        with np.errstate(divide="ignore", over="ignore"):   # 1/sqrt(0), results beyond fp32
            want = (1.0 / np.sqrt(ss / np.float64(cols) + e64)).astype(np.float32)
        bad = np.flatnonzero(got.view(np.uint32) != want.view(np.uint32))
        assert bad.size == 0, (name, [(float(ss[i]), float(got[i]), float(want[i])) for i in bad[:5]])
        share = float(fast.mean())
        print(f"[sweep] inverse RMS {name}: {ss.size} values, fast path {share:.6f}", flush=True)
        if name == "random":
            assert share >= 0.9999
        elif name == "midpoint":
            assert share <= 0.01


# instruction kinds of the issue-rate probe, in its numbering, with the
# independent chains each lane runs
_ISSUE_KINDS = [("fp32 FMA", 8), ("exp2 (transcendental)", 8), ("rcp (transcendental)", 8),
                ("v_cvt_pk_bf16_f32", 8), ("v_cvt_pk_fp8_f32", 8), ("v_bitop3_b32", 8),
                ("integer add", 8), ("fp64 FMA", 4), ("v_dot2c_f32_bf16", 8)]


def test_issue_rates():
    """The issue rate of each instruction kind the kernels' arithmetic is
    built from: a register-only kernel per kind (8 independent chains a lane,
    4096 blocks of 256 lanes), timed by events, in cycles per wave64
    instruction per SIMD at the nominal 2.4 GHz.  The figures are printed
    (pytest -s shows them); the test asserts only that every kernel ran."""
    L = _probe()
    blocks, n = 4096, 4000
    out = torch.empty(blocks * 256, dtype=torch.int32, device="cuda")
    simds = 4 * torch.cuda.get_device_properties(0).multi_processor_count
    assert L.afqp_issue(0, out.data_ptr(), blocks, n, _stream()) == 0   # warm-up
    torch.cuda.synchronize()
    print(f"\nissue rates ({simds} SIMDs, 2.4 GHz nominal):", flush=True)
    for op, (name, chains) in enumerate(_ISSUE_KINDS):
        ms = []
        for _ in range(3):
            s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            s.record()
            rc = L.afqp_issue(op, out.data_ptr(), blocks, n, _stream())
            e.record()
            torch.cuda.synchronize()
            assert rc == 0, (name, rc)
            ms.append(s.elapsed_time(e))
        t = sorted(ms)[1]
        assert t > 0
        cycles = t * 1e-3 * simds * 2.4e9 / (blocks * 4 * n * chains)
        print(f"  {name:24s} {cycles:5.2f} cycles per wave64 instruction per SIMD", flush=True)
