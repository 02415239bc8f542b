"""The fp32-scale quantiser's slow path on the GPU (1x128 and per-token).

Group maxima below 2^-83 leave the fast path (a corrected product for the
scale, a corrected hardware reciprocal and a corrected quotient): the scale
and every quotient are IEEE divisions followed by the clamp.  Below
448 * 2^-126 the scale is an fp32 subnormal, and at or below 224 * 2^-149
it underflows to 0, which gives all-zero codes (reading R25).  These tests
put group maxima on both sides of each boundary (and of 2^-116, where the
scale alone would still be exact) and deep in the subnormal range, through
the standalone quantiser (bf16 and fp32 rows) and through the norm
(standard RMSNorm whose weights are tiny, so that the normed rows are), and
compare with the oracle.  Tiny-amax groups are the "tiny" blocks of [P1]
"Test Plan / Correctness"."""
import numpy as np
import pytest
import torch

import activation_fp8_quant_amd as afq
import oracle as orc
from activation_fp8_quant_amd import inputs
from tests._gpu import HOST_THREADS, MODE, check_norm, dev16, host8, host16, ref_norm, run_norm, scales_u8_or_f32

pytestmark = pytest.mark.gpu

BOUND_FAST = 2.0 ** -83           # fast path from here up
BOUND_SCALE = 2.0 ** -116         # the fast scale alone would be exact from here up
BOUND_NORMAL = 448.0 * 2.0 ** -126  # the scale is an fp32 normal from here up
BOUND_ZERO = 224.0 * 2.0 ** -149  # the scale underflows to 0 at and below this


def _f32_neighbours(x: float, k: int = 3) -> np.ndarray:
    """x and the k fp32 values on either side of it."""
    b = int(np.float32(x).view(np.uint32))
    return np.arange(b - k, b + k + 1, dtype=np.uint32).view(np.float32)


def _bf16_neighbours(x: float, k: int = 2) -> np.ndarray:
    b = int(inputs.to_bits(np.array([x]))[0])
    bits = np.arange(b - k, b + k + 1, dtype=np.uint16)
    return inputs.bits_to_float(bits)


def _amax_list(dtype: str) -> np.ndarray:
    if dtype == "fp32":
        vals = [_f32_neighbours(BOUND_FAST), _f32_neighbours(BOUND_SCALE), _f32_neighbours(BOUND_NORMAL),
                _f32_neighbours(BOUND_ZERO),
                np.array([2.0 ** -126, 1e-39, 3e-42, 2.0 ** -149, 2.0 ** -110, 1.0], np.float32)]
    else:
        vals = [_bf16_neighbours(BOUND_FAST), _bf16_neighbours(BOUND_SCALE), _bf16_neighbours(BOUND_NORMAL),
                np.array([2.0 ** -126, 2.0 ** -130, 2.0 ** -133, 2.0 ** -110, 1.0], np.float32)]
    return np.concatenate(vals).astype(np.float32)


def _rows(amaxes: np.ndarray, width: int, group: int, rng) -> np.ndarray:
    """One row per amax: every group of `group` elements has largest
    magnitude amax (at a random position, random sign); the others are
    random fractions of it (down into the subnormals)."""
    M = amaxes.size
    x = rng.uniform(-1, 1, (M, width)) * amaxes[:, None].astype(np.float64)
    x *= 2.0 ** -rng.integers(0, 12, (M, width))
    g = x.reshape(M, width // group, group)
    pos = rng.integers(0, group, (M, width // group))
    sgn = np.where(rng.random((M, width // group)) < 0.5, -1.0, 1.0)
    np.put_along_axis(g, pos[..., None], (sgn * amaxes[:, None])[..., None], axis=2)
    return g.reshape(M, width)


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("mode,width", [("b128", 256), ("pt", 256), ("pt", 6144), ("b128", 6144)])
def test_quant_tiny_amax_around_both_boundaries(dtype, mode, width):
    """fp8_quant (1x128, per-token) on rows whose group maxima straddle
    2^-83, 2^-116, 448 * 2^-126 and (fp32) 224 * 2^-149 (a few values either
    side) and lie deep in the subnormals: codes and scales bit-exact against
    the oracle."""
    rng = np.random.default_rng(61)
    am = _amax_list(dtype)
    group = 128 if mode == "b128" else width
    x = _rows(am, width, group, rng)
    if dtype == "fp32":
        xh = x.astype(np.float32)
        # the group maxima exactly as chosen (fp32 rounding of the fractions
        # cannot exceed them)
        xt = torch.from_numpy(xh).cuda()
        odt = orc.FP32
    else:
        xh = inputs.to_bits(x, "bf16")
        xt = dev16(xh)
        odt = orc.BF16
    print(f"case tiny-amax quant {mode} {dtype} width={width} rows={am.size}", flush=True)
    qa = afq.fp8_quant(xt, MODE[mode])
    torch.cuda.synchronize()
    q, s = orc.quant(xh, odt, MODE[mode], threads=HOST_THREADS)
    assert np.array_equal(scales_u8_or_f32(qa.scales).view(np.uint32), s.view(np.uint32))
    bad = np.argwhere(host8(qa.values) != q)
    assert bad.size == 0, [(float(x[tuple(b)]), int(host8(qa.values)[tuple(b)]), int(q[tuple(b)]))
                           for b in bad[:5]]
    # both sides of the boundaries are present among the group maxima
    s32 = s.ravel()
    slow = s32 < np.float32(BOUND_FAST / 448)
    assert slow.any() and (~slow).any() and (s32 < np.float32(2.0 ** -126)).any() and \
        ((s32 >= np.float32(2.0 ** -126)) & slow).any()
    if dtype == "fp32":
        assert (s32 == 0).any() and (s32 > 0).any()


@pytest.mark.parametrize("qin", [0, 1])
@pytest.mark.parametrize("mode", ["b128", "pt"])
@pytest.mark.parametrize("M,H", [(64, 4096), (300, 4096), (9, 2048), (300, 2048), (300, 1024)])
def test_norm_tiny_weights_slow_path(qin, mode, M, H):
    """Standard RMSNorm whose weights are U(0.5, 1.5) * 2^k (k = -85,
    -118, -119, -120, -124): the normed rows are tiny, so group maxima fall
    on both sides of 2^-83, of 2^-116 and of 448 * 2^-126 and below; 1x128
    and per-token, at decode and bandwidth row shapes (per-token rows of
    2048 and 1024 at 300 rows run one wavefront a row), the default and the
    fp32-direct quantiser input.  Against the oracle within the contract
    (fp32-direct: bit-exact)."""
    d = inputs.norm_inputs(M, H, seed=62, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    w = inputs.bits_to_float(d["w"], "bf16").astype(np.float64)
    seen_slow = seen_sub = 0
    for k in (-85, -118, -119, -120, -124):
        wk = inputs.to_bits(w * 2.0 ** k)
        print(f"case tiny-weight norm {mode} qin={qin} M={M} H={H} k={k}", flush=True)
        gpu = run_norm(d["x"], wk, r=d["r"], kind="standard", mode=mode, qin=qin)
        ref = ref_norm(d["x"], wk, r=d["r"], kind="standard", mode=mode, qin=qin)
        check_norm(gpu, ref, mode, "bf16", f"tiny-w {mode} k={k}", requant=(qin == 0), qin=qin)
        s = np.asarray(ref["scales"], np.float32).ravel()
        seen_slow += int(((s > 0) & (s < np.float32(BOUND_FAST / 448))).sum())
        seen_sub += int(((s > 0) & (s < np.float32(2.0 ** -126))).sum())
    assert seen_slow > 0 and seen_sub > 0


@pytest.mark.parametrize("M", [8, 300])
@pytest.mark.parametrize("tiny", [0, 1])
def test_two_segments_one_on_the_slow_path(M, tiny):
    """Two per-token segments (1536 + 512) where one segment's weights are
    scaled by 2^-120 (its scale on the slow path) and the
    other's are not: the per-row choice between the fast and the slow
    quantiser must follow each segment, at 8 and 300 rows (one wavefront a
    row); against the oracle."""
    segs = inputs.two_segment_inputs(M, (1536, 512), seed=63)
    w = inputs.bits_to_float(segs[tiny]["w"], "bf16").astype(np.float64)
    segs[tiny]["w"] = inputs.to_bits(w * 2.0 ** -120)
    print(f"case two segments, segment {tiny} tiny, M={M}", flush=True)
    outs = afq.fused_add_rmsnorm_quant([dev16(sg["x"]) for sg in segs], [dev16(sg["w"]) for sg in segs], 1e-6,
                                       mode=afq.PER_TOKEN, kind=afq.STANDARD, want_normed=True)
    torch.cuda.synchronize()
    for j, (sg, qa) in enumerate(zip(segs, outs)):
        gpu = dict(normed=host16(qa.normed), values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(sg["x"], sg["w"], kind="standard", mode="pt")
        check_norm(gpu, ref, "pt", "bf16", f"two-seg tiny={tiny} seg {j} M={M}")
        s = np.asarray(ref["scales"], np.float32).ravel()
        if j == tiny:
            assert bool((s < np.float32(BOUND_FAST / 448)).all())
        else:
            assert bool((s >= np.float32(BOUND_FAST / 448)).all())
