"""GPU parity: the HIP kernels (through the C ABI) against the CPU oracle,
element by element on seeded inputs shaped like the pages' workloads, at
sizes spanning several tiles and a ragged tail, plus edge rows."""
import numpy as np
import pytest
import torch

import activation_fp8_quant_amd as afq
import oracle as orc
from activation_fp8_quant_amd import inputs
from tests._compare import check_codes, check_dtype16, check_scales, scales_u8_or_f32
from tests._gpu import (HOST_THREADS, MODE, ORC_DT, check_norm, dev16, host8, host16, ref_norm,
                        run_norm)

pytestmark = pytest.mark.gpu


def _report(name, stats):
    print(f"[parity] {name}: {stats}", flush=True)


# ------------------------------------------------------------ norm paths
@pytest.mark.parametrize("M", [8, 67])
def test_norm_gemma_mx_h6144(M):
    """Fused add + Gemma RMSNorm + MXFP8 + bf16 copy at the decode shape
    (hidden 6144): x ~ N(0,3^2), r ~ N(0,1), w ~ N(0,0.1^2), eps 1e-6."""
    d = inputs.norm_inputs(M, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode="mx")
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode="mx")
    _report(f"gemma-mx M={M}", check_norm(gpu, ref, "mx", "bf16", "gemma-mx"))


@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
@pytest.mark.parametrize("kind", ["gemma", "standard"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("H,M", [(6144, 17), (4096, 33), (2048, 5), (1024, 130), (512, 9)])
def test_norm_modes(mode, kind, dtype, H, M):
    d = inputs.norm_inputs(M, H, seed=3, x_std=1.0, r_std=1.0,
                           w_kind="uniform" if kind == "standard" else "normal",
                           w_param=0.5 if kind == "standard" else 0.1, dtype=dtype)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode, dtype=dtype)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode, dtype=dtype)
    _report(f"{mode}-{kind}-{dtype} H={H} M={M}", check_norm(gpu, ref, mode, dtype, "norm"))


@pytest.mark.parametrize("H", [2176, 7168, 12288, 20480, 24576, 32768, 128, 8])
def test_norm_widths(H):
    mode = "b128" if H % 128 == 0 else "pt"
    d = inputs.norm_inputs(7, H, seed=4, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="standard", mode=mode)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode=mode)
    _report(f"width {H} {mode}", check_norm(gpu, ref, mode, "bf16", f"width{H}"))
    if H % 32 == 0:
        gpu = run_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="mx")
        ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="mx")
        check_norm(gpu, ref, "mx", "bf16", f"width{H}-mx")


def test_norm_without_residual_and_without_copy():
    d = inputs.norm_inputs(20, 4096, seed=5, x_std=1.0, r_std=None, w_kind="uniform", w_param=0.5)
    for mode in ("mx", "b128", "pt"):
        gpu = run_norm(d["x"], d["w"], kind="standard", mode=mode, want_normed=False)
        ref = ref_norm(d["x"], d["w"], kind="standard", mode=mode)
        check_codes(gpu["values"], ref["values"], mode)
        check_scales(gpu["scales"], ref["scales"], MODE[mode], mode, u=ref["normed"], dtype="bf16")


def test_norm_inplace_residual():
    d = inputs.norm_inputs(16, 6144, seed=6, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    xt, wt, rt = dev16(d["x"]), dev16(d["w"]), dev16(d["r"])
    qa = afq.fused_add_rmsnorm_quant(xt, wt, 1e-6, mode=afq.MXFP8, kind=afq.GEMMA, residual=rt,
                                     inplace=True, want_normed=True)
    torch.cuda.synchronize()
    assert qa.residual.data_ptr() == rt.data_ptr()
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode="mx")
    check_dtype16(host16(rt), ref["h"], "inplace h", exact=True)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
def test_norm_edge_rows(mode, dtype):
    """The edge rows in both dtypes (in fp16 the tiny row underflows to zero
    and the dominated row's small entries become fp16 subnormals)."""
    H = 2048
    rows = inputs.edge_rows(H)
    x = inputs.to_bits(rows, dtype)
    r = inputs.to_bits(np.zeros_like(rows), dtype)
    w = inputs.to_bits(np.random.default_rng(3).uniform(0.5, 1.5, H), dtype)
    for kind in ("standard", "gemma"):
        gpu = run_norm(x, w, r=r, kind=kind, mode=mode, dtype=dtype)
        ref = ref_norm(x, w, r=r, kind=kind, mode=mode, dtype=dtype)
        _report(f"edge {mode} {kind} {dtype}",
                check_norm(gpu, ref, mode, dtype, f"edge-{mode}-{kind}-{dtype}"))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M", [1, 8, 64, 1024])
def test_two_segment_per_token(dtype, M):
    """q [M,1536] and kv [M,512] normed in one launch with separate weights,
    per-token scales each; inputs with 1 % x50 outliers; q and kv are column
    slices of one [M, 2112] buffer (the fused qkv_a projection output)."""
    segs = inputs.two_segment_inputs(M, (1536, 512), seed=0, dtype=dtype)
    buf = np.zeros((M, 2112), np.uint16)
    buf[:, :1536] = segs[0]["x"]
    buf[:, 1536:2048] = segs[1]["x"]
    bt = dev16(buf, dtype)
    xq, xkv = bt[:, :1536], bt[:, 1536:2048]
    wq, wkv = dev16(segs[0]["w"], dtype), dev16(segs[1]["w"], dtype)
    outs = afq.fused_add_rmsnorm_quant([xq, xkv], [wq, wkv], 1e-6, mode=afq.PER_TOKEN,
                                       kind=afq.STANDARD, want_normed=True)
    torch.cuda.synchronize()
    for s, qa in zip(segs, outs):
        assert qa.orig_dtype == (torch.bfloat16 if dtype == "bf16" else torch.float16)
        gpu = dict(normed=host16(qa.normed), values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(s["x"], s["w"], kind="standard", mode="pt", dtype=dtype)
        _report(f"two-seg {dtype} M={M} cols={s['x'].shape[1]}", check_norm(gpu, ref, "pt", dtype, "two-seg"))


@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
@pytest.mark.parametrize("H", [4096, 6144])
def test_norm_bandwidth_row_counts(mode, H):
    """1100 rows: the per-token launch takes two (width 4096) or three (6144)
    chunks per lane, the MXFP8 launch with the copy two (1x128 one): every
    row against the oracle."""
    M = 1100
    d = inputs.norm_inputs(M, H, seed=8, x_std=2.0, r_std=1.0, w_kind="normal", w_param=0.1)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode=mode)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode=mode)
    _report(f"bandwidth rows {mode} H={H}", check_norm(gpu, ref, mode, "bf16", f"bw-{mode}"))


@pytest.mark.parametrize("mode,H,M,dtype", [
    ("mx", 6144, 1536, "bf16"),   # three chunks per lane
    ("mx", 4096, 3072, "bf16"),   # four chunks per lane, two rows of 128 lanes per block
    ("mx", 8192, 1536, "fp16"),   # four chunks per lane, 256 lanes
    ("mx", 2048, 3072, "bf16"),   # two chunks per lane, two rows per block
    ("mx", 2048, 2048, "bf16"),   # a full round at one chunk per lane: two, two rows per block
    ("mx", 8192, 512, "fp16"),    # a full round at one chunk per lane: two, 512 lanes
    ("mx", 4096, 2048, "fp16"),   # a full round at two: four chunks per lane, two rows per block
    ("mx", 7168, 1536, "bf16"),   # four chunks per lane on 256 lanes (128 idle chunk slots)
    ("pt", 6144, 300, "bf16"),    # above 256 rows: three chunks per lane
    ("pt", 8192, 64, "fp16"),     # up to 256 rows: two chunks per lane, 512 lanes
    ("pt", 2048, 257, "bf16"),    # two chunks per lane, two rows per block, a ragged block
    ("mx", 16384, 600, "bf16"),   # wider than 1024 chunks: base two per lane, one round at four
    ("mx", 8224, 1000, "bf16"),   # 1028 chunks: base two per lane (576 lanes), one round at three
    ("pt", 16384, 300, "fp16"),   # per-token above 256 rows at two chunks per lane, 1024 lanes
])
def test_norm_row_shapes_by_size(mode, H, M, dtype):
    """The row shapes the launcher picks by row count (MXFP8 with the copy
    wherever one round of the base shape cannot hold every row with room to
    spare, up to three rounds; per-token at every size): every row against
    the oracle, with the copy."""
    print(f"case row shape {mode} H={H} M={M} {dtype}", flush=True)
    d = inputs.norm_inputs(M, H, seed=13, x_std=2.0, r_std=1.0, w_kind="normal", w_param=0.1,
                           dtype=dtype)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode=mode, dtype=dtype)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode=mode, dtype=dtype)
    _report(f"row shape {mode} H={H} M={M}", check_norm(gpu, ref, mode, dtype, f"shape-{mode}"))


@pytest.mark.parametrize("mode,H,Ms,qin", [
    ("pt", 6144, (8, 300, 1100), 0),     # 2, 3, 3 chunks per lane
    ("pt", 2048, (8, 300, 1100), 0),     # 1 chunk per lane, then one wavefront a row (4 per lane)
    ("pt", 8192, (8, 300), 1),           # fp32-direct: 2 chunks per lane, 512 then 512 lanes
    ("mx", 6144, (8, 1024, 1536), 0),    # 1, 2, 3 chunks per lane
    ("mx", 4096, (8, 1536, 3072), 0),    # 1, 2, 4 chunks per lane (two rows per block)
    ("b128", 4096, (8, 1100), 1),        # fp32-direct 1x128: 1 chunk per lane
    ("mx", 16384, (8, 600, 1000), 0),    # 2 (1024 lanes), 4 (512 lanes), 2 chunks per lane
])
def test_rows_independent_of_launch_shape(mode, H, Ms, qin):
    """The row shape depends on the row count, but the mean square is summed
    in an order fixed by the width: the first 8 rows come out bit-identical
    from launches of every row count and from the copy-only launch (one
    chunk per lane), residual and copy included."""
    print(f"case shape invariance {mode} H={H} Ms={Ms} qin={qin}", flush=True)
    Mmax = max(Ms)
    d = inputs.norm_inputs(Mmax, H, seed=17, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    first = None
    for M in Ms:
        g = run_norm(d["x"][:M], d["w"], r=d["r"][:M], kind="gemma", mode=mode, qin=qin)
        rows = {k: np.ascontiguousarray(g[k][:8]) for k in ("h", "normed", "values", "scales")}
        if first is None:
            first = rows
            ref = ref_norm(d["x"][:8], d["w"], r=d["r"][:8], kind="gemma", mode=mode, qin=qin)
            check_norm(g, ref, mode, "bf16", f"shape-inv-{mode}", requant=(qin == 0), qin=qin)
        for k in rows:
            assert np.array_equal(rows[k], first[k]), (M, k)
    x, w, r = dev16(d["x"][:300]), dev16(d["w"]), dev16(d["r"][:300])
    plain = afq.fused_add_rmsnorm_quant(x, w, 1e-6, mode=MODE[mode], kind=afq.GEMMA, residual=r,
                                        quantize=False)
    torch.cuda.synchronize()
    if qin == 0:
        assert np.array_equal(host16(plain.normed)[:8], first["normed"])
    assert np.array_equal(host16(plain.residual)[:8], first["h"])


@pytest.mark.parametrize("H", [20480, 32768])
def test_per_token_wide_rows_bandwidth_shape(H):
    """Per-token rows above 1024 rows take at least two chunks per lane, and
    wide rows more (three at 20480, four at 32768): 1030 rows, every row
    against the oracle, fp16."""
    d = inputs.norm_inputs(1030, H, seed=42, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5,
                           dtype="fp16")
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="pt", dtype="fp16")
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="pt", dtype="fp16")
    _report(f"per-token wide H={H}", check_norm(gpu, ref, "pt", "fp16", f"pt-wide{H}"))


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("M,copy", [(2048, True), (8192, False)])
def test_two_segment_bandwidth_row_counts(M, copy, dtype):
    """The two-segment per-token launch above 1024 rows, every row against
    the oracle; M = 8192 is the benchmark workload, launched exactly as
    timed (no copy), in both dtypes."""
    print(f"case two-seg bandwidth M={M} {dtype} copy={copy}", flush=True)
    segs = inputs.two_segment_inputs(M, (1536, 512), seed=0, dtype=dtype)
    buf = np.zeros((M, 2112), np.uint16)
    buf[:, :1536] = segs[0]["x"]
    buf[:, 1536:2048] = segs[1]["x"]
    bt = dev16(buf, dtype)
    outs = afq.fused_add_rmsnorm_quant([bt[:, :1536], bt[:, 1536:2048]],
                                       [dev16(segs[0]["w"], dtype), dev16(segs[1]["w"], dtype)], 1e-6,
                                       mode=afq.PER_TOKEN, kind=afq.STANDARD, want_normed=copy)
    torch.cuda.synchronize()
    for s, qa in zip(segs, outs):
        gpu = dict(normed=host16(qa.normed) if copy else None, values=host8(qa.values),
                   scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(s["x"], s["w"], kind="standard", mode="pt", dtype=dtype)
        _report(f"two-seg bandwidth M={M} {dtype} cols={s['x'].shape[1]}",
                check_norm(gpu, ref, "pt", dtype, "two-seg-bw"))


def test_two_segment_other_modes():
    segs = inputs.two_segment_inputs(12, (1536, 512), seed=2)
    for mode in ("mx", "b128"):
        xs = [dev16(s["x"]) for s in segs]
        ws = [dev16(s["w"]) for s in segs]
        outs = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=MODE[mode], kind=afq.STANDARD,
                                           want_normed=True)
        torch.cuda.synchronize()
        for s, qa in zip(segs, outs):
            gpu = dict(normed=host16(qa.normed), values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))
            ref = ref_norm(s["x"], s["w"], kind="standard", mode=mode)
            check_norm(gpu, ref, mode, "bf16", f"two-seg-{mode}")


@pytest.mark.parametrize("mode,widths,qin", [("pt", (1000, 512), 0), ("pt", (8, 2040), 0),
                                             ("mx", (1568, 512), 0), ("b128", (1664, 384), 0),
                                             ("pt", (1000, 512), 1), ("b128", (1664, 384), 1)])
@pytest.mark.parametrize("M", [7, 1100])
def test_two_segment_unaligned_boundary(mode, widths, qin, M):
    """Two segments whose boundary is not on a 64-chunk line (the first
    segment's chunk count is not a multiple of 64, down to a single chunk),
    so the segment of each chunk is chosen per lane; at a decode row count
    and at the bandwidth-bound row shape, with the default and the
    fp32-direct quantiser input."""
    segs = inputs.two_segment_inputs(M, widths, seed=41)
    xs = [dev16(sg["x"]) for sg in segs]
    ws = [dev16(sg["w"]) for sg in segs]
    outs = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=MODE[mode], kind=afq.STANDARD,
                                       want_normed=True, quant_input=qin)
    torch.cuda.synchronize()
    for sg, qa in zip(segs, outs):
        gpu = dict(normed=host16(qa.normed), values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(sg["x"], sg["w"], kind="standard", mode=mode, qin=qin)
        name = f"two-seg {widths} {mode} qin={qin} M={M}"
        _report(name, check_norm(gpu, ref, mode, "bf16", name, requant=(qin == 0), qin=qin))


@pytest.mark.parametrize("widths,dtype", [((1536, 512), "bf16"), ((1536, 512), "fp16"), ((512, 1536), "bf16"),
                                          ((1024, 1024), "bf16"), ((1000, 512), "bf16"), ((8, 2040), "bf16")])
def test_two_segment_rows_independent_of_launch_shape(widths, dtype):
    """Two per-token segments on one wavefront a row, with the segment
    boundary in slot 3, 1 or 2 (1536 + 512, 512 + 1536, 1024 + 1024) or
    inside a slot (1000 + 512, 8 + 2040), at 8, 300 and 1100 rows: the first
    8 rows of every launch are bit-identical (codes, scales, copy), and
    against the oracle; and their copy equals, bit for bit, the copy-only
    launch of the same rows, which runs the multi-wavefront kernel (one
    chunk per lane, the rows' sums of squares meeting in LDS)."""
    print(f"case two-seg shape invariance {widths} {dtype}", flush=True)
    segs = inputs.two_segment_inputs(1100, widths, seed=43, dtype=dtype)
    first = None
    for M in (8, 300, 1100):
        xs = [dev16(sg["x"][:M], dtype) for sg in segs]
        ws = [dev16(sg["w"], dtype) for sg in segs]
        outs = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=afq.PER_TOKEN, kind=afq.STANDARD,
                                           want_normed=True)
        torch.cuda.synchronize()
        rows = [dict(normed=host16(qa.normed)[:8], values=host8(qa.values)[:8],
                     scales=scales_u8_or_f32(qa.scales)[:8]) for qa in outs]
        if first is None:
            first = rows
            for sg, g in zip(segs, rows):
                ref = ref_norm(sg["x"][:8], sg["w"], kind="standard", mode="pt", dtype=dtype)
                check_norm(g, ref, "pt", dtype, f"two-seg-shape {widths}")
        for i, (a, b) in enumerate(zip(rows, first)):
            for k in a:
                assert np.array_equal(np.asarray(a[k]).view(np.uint8), np.asarray(b[k]).view(np.uint8)), \
                    (widths, M, i, k)
    xs = [dev16(sg["x"][:8], dtype) for sg in segs]
    ws = [dev16(sg["w"], dtype) for sg in segs]
    plain = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=afq.PER_TOKEN, kind=afq.STANDARD,
                                        quantize=False)
    torch.cuda.synchronize()
    for i, (qa, b) in enumerate(zip(plain, first)):
        assert np.array_equal(host16(qa.normed), b["normed"]), (widths, i)


# ----------------------------------------------------------- SiLU-and-mul
def _random_norm_configs(n, seed, budget=1.2e8):
    """n seeded random norm launches: mode, kind, dtype, width (log-uniform
    over 8-element chunks, a multiple of the group), row count (log-uniform
    in 1 .. 6000), residual, copy, quantiser input and one or two segments;
    at most `budget` elements in all, so the oracle runs in seconds."""
    rng = np.random.default_rng(seed)
    out, total = [], 0
    for _ in range(1_000_000):
        if len(out) == n:
            break
        mode = str(rng.choice(["mx", "b128", "pt"]))
        g = {"mx": 4, "b128": 16, "pt": 1}[mode]             # group in chunks
        nseg = 2 if rng.random() < 0.25 else 1
        widths = []
        for _ in range(nseg):
            c = int(np.exp(rng.uniform(0.0, np.log(4096 // nseg))))
            widths.append(8 * max(g, c // g * g))
        M = int(np.exp(rng.uniform(0.0, np.log(6000))))
        elems = M * sum(widths)
        if elems > 3e7 or total + elems > budget:
            continue
        total += elems
        out.append(dict(mode=mode, widths=tuple(widths), M=M, kind=str(rng.choice(["gemma", "standard"])),
                        dtype=str(rng.choice(["bf16", "fp16"])), res=nseg == 1 and rng.random() < 0.7,
                        copy=bool(rng.random() < 0.7),
                        qin=1 if mode != "mx" and rng.random() < 0.25 else 0, seed=int(rng.integers(1 << 30))))
    if len(out) < n:
        raise RuntimeError(f"{n} configurations do not fit a budget of {budget:g} elements")
    return out


@pytest.mark.parametrize("cfg", _random_norm_configs(32, seed=20261203),
                         ids=lambda c: f"{c['mode']}-{'+'.join(map(str, c['widths']))}-M{c['M']}-{c['kind']}-{c['dtype']}"
                                       f"{'-res' if c['res'] else ''}{'-copy' if c['copy'] else ''}{'-f32q' if c['qin'] else ''}")
def test_norm_random_configurations(cfg):
    """Seeded random launches over every option of the norm (mode, kind,
    dtype, width, row count, residual, copy, quantiser input, one or two
    segments), so that the row-shape rules are reached at widths and row
    counts no other test picks: every row against the oracle."""
    print(f"case random norm {cfg}", flush=True)
    mode, dtype, kind, qin = cfg["mode"], cfg["dtype"], cfg["kind"], cfg["qin"]
    w_kind, w_param = ("normal", 0.1) if kind == "gemma" else ("uniform", 0.5)
    if len(cfg["widths"]) == 1:
        H = cfg["widths"][0]
        d = inputs.norm_inputs(cfg["M"], H, seed=cfg["seed"], x_std=3.0, r_std=1.0 if cfg["res"] else None,
                               w_kind=w_kind, w_param=w_param, dtype=dtype)
        gpu = run_norm(d["x"], d["w"], r=d.get("r"), kind=kind, mode=mode, dtype=dtype,
                       want_normed=cfg["copy"], qin=qin)
        ref = ref_norm(d["x"], d["w"], r=d.get("r"), kind=kind, mode=mode, dtype=dtype, qin=qin)
        check_norm(gpu, ref, mode, dtype, f"random {cfg}", requant=qin == 0, qin=qin)
        return
    segs = inputs.two_segment_inputs(cfg["M"], cfg["widths"], seed=cfg["seed"], dtype=dtype)
    xs = [dev16(sg["x"], dtype) for sg in segs]
    ws = [dev16(sg["w"], dtype) for sg in segs]
    outs = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=MODE[mode], kind=afq.GEMMA if kind == "gemma" else afq.STANDARD,
                                       want_normed=cfg["copy"], quant_input=qin)
    torch.cuda.synchronize()
    for sg, qa in zip(segs, outs):
        gpu = dict(normed=host16(qa.normed) if cfg["copy"] else None, values=host8(qa.values),
                   scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(sg["x"], sg["w"], kind=kind, mode=mode, dtype=dtype, qin=qin)
        check_norm(gpu, ref, mode, dtype, f"random {cfg}", requant=qin == 0, qin=qin)


def _random_act_configs(n, seed, budget=1.0e8):
    """n seeded random activation launches: SiLU-and-mul in MXFP8 (with or
    without the bf16 copy, the default or the bf16-first quantiser input)
    or 1x128, or the clamped SwiGLU in MXFP8; width I log-uniform over
    groups, rows log-uniform in 1 .. 6000, gate/up spread N(0, s^2) with s in
    {1, 2, 3, 8}; at most `budget` activations in all."""
    rng = np.random.default_rng(seed)
    out, total = [], 0
    for _ in range(1_000_000):
        if len(out) == n:
            break
        act = str(rng.choice(["silu", "silu", "swiglu"]))
        mode = "mx" if act == "swiglu" else str(rng.choice(["mx", "b128"]))
        g = 32 if mode == "mx" else 128
        I = g * max(1, int(np.exp(rng.uniform(0.0, np.log(16384 // g)))))
        M = int(np.exp(rng.uniform(0.0, np.log(6000))))
        if M * I > 2e7 or total + M * I > budget:
            continue
        total += M * I
        out.append(dict(act=act, mode=mode, I=I, M=M, std=float(rng.choice([1.0, 2.0, 3.0, 8.0])),
                        copy=bool(rng.random() < 0.5), qin=2 if mode == "mx" and rng.random() < 0.3 else 0,
                        seed=int(rng.integers(1 << 30))))
    if len(out) < n:
        raise RuntimeError(f"{n} configurations do not fit a budget of {budget:g} activations")
    return out


@pytest.mark.parametrize("cfg", _random_act_configs(24, seed=20261204),
                         ids=lambda c: f"{c['act']}-{c['mode']}-I{c['I']}-M{c['M']}-s{c['std']:g}"
                                       f"{'-copy' if c['copy'] else ''}{'-bf16first' if c['qin'] else ''}")
def test_activation_random_configurations(cfg):
    """Seeded random SiLU-and-mul / clamped SwiGLU launches over mode, width,
    row count, input spread, copy and quantiser input (so both forms of the
    MXFP8 kernel, four values a lane and eight, are reached at widths no
    other test picks): every row against the oracle, 1x128 bit-exact."""
    print(f"case random activation {cfg}", flush=True)
    gu = inputs.gate_up_inputs(cfg["M"], cfg["I"], seed=cfg["seed"], std=cfg["std"])
    gt = dev16(gu)
    if cfg["act"] == "swiglu":
        qa = afq.swiglu_oai_quant(gt, 1.702, 1.0, 7.0, want_act=cfg["copy"], quant_input=cfg["qin"])
        ref = orc.swiglu_oai_quant(gu, 1.702, 1.0, 7.0, orc.MXFP8, threads=HOST_THREADS, qin=cfg["qin"])
    else:
        qa = afq.silu_mul_quant(gt, MODE[cfg["mode"]], want_act=cfg["copy"], quant_input=cfg["qin"])
        ref = orc.silu_quant(gu, MODE[cfg["mode"]], threads=HOST_THREADS, qin=cfg["qin"])
    torch.cuda.synchronize()
    values, scales = host8(qa.values), scales_u8_or_f32(qa.scales)
    name = f"random {cfg}"
    if cfg["mode"] == "b128":
        assert np.array_equal(values, ref["values"]), name
        assert np.array_equal(scales.view(np.uint32), ref["scales"].view(np.uint32)), name
        if cfg["copy"]:
            check_dtype16(host16(qa.normed), ref["act"], name + " act", exact=True)
        return
    check_codes(values, ref["values"], name)
    check_scales(scales, ref["scales"], 0, name)
    if cfg["copy"]:
        check_dtype16(host16(qa.normed), ref["act"], name + " act")
        if cfg["qin"] == 2:   # bf16-first: the fused codes are the quantiser's of the kernel's own copy
            sep = afq.fp8_quant(qa.normed, afq.MXFP8)
            torch.cuda.synchronize()
            assert np.array_equal(values, host8(sep.values)), name
            assert np.array_equal(scales, scales_u8_or_f32(sep.scales)), name


def _random_quant_configs(n, seed, budget=1.0e8):
    """n seeded random standalone quantiser launches: mode, input dtype
    (bf16, fp16, fp32), width log-uniform over groups, rows log-uniform in
    1 .. 6000, rows scaled by 2^k with k in [-40, 40]; at most `budget`
    elements in all."""
    rng = np.random.default_rng(seed)
    out, total = [], 0
    for _ in range(1_000_000):
        if len(out) == n:
            break
        mode = str(rng.choice(["mx", "b128", "pt"]))
        g = {"mx": 32, "b128": 128, "pt": 8}[mode]
        cols = g * max(1, int(np.exp(rng.uniform(0.0, np.log(32768 // g)))))
        M = int(np.exp(rng.uniform(0.0, np.log(6000))))
        if M * cols > 2e7 or total + M * cols > budget:
            continue
        total += M * cols
        out.append(dict(mode=mode, dtype=str(rng.choice(["bf16", "fp16", "fp32"])), cols=cols, M=M,
                        seed=int(rng.integers(1 << 30))))
    if len(out) < n:
        raise RuntimeError(f"{n} configurations do not fit a budget of {budget:g} elements")
    return out


@pytest.mark.parametrize("cfg", _random_quant_configs(24, seed=20261205),
                         ids=lambda c: f"{c['mode']}-{c['dtype']}-{c['cols']}-M{c['M']}")
def test_fp8_quant_random_configurations(cfg):
    """Seeded random standalone quantiser launches (every mode and input
    dtype, widths up to 32768, row counts that reach each per-token row
    shape, rows spread over 80 binades): codes and scales bit-exact."""
    print(f"case random quant {cfg}", flush=True)
    rng = np.random.default_rng(cfg["seed"])
    M, n, dtype = cfg["M"], cfg["cols"], cfg["dtype"]
    x = rng.standard_normal((M, n)) * 2.0 ** rng.integers(-40, 41, (M, 1))
    if dtype == "fp16":
        x = np.clip(x, -60000.0, 60000.0)
    if dtype == "fp32":
        xh = x.astype(np.float32)
        xt = torch.from_numpy(xh).cuda()
        odt = orc.FP32
    else:
        xh = inputs.to_bits(x, dtype)
        xt = dev16(xh, dtype)
        odt = ORC_DT[dtype]
    qa = afq.fp8_quant(xt, MODE[cfg["mode"]])
    torch.cuda.synchronize()
    q, s = orc.quant(xh, odt, MODE[cfg["mode"]], threads=HOST_THREADS)
    assert np.array_equal(host8(qa.values), q), cfg
    gs = scales_u8_or_f32(qa.scales)
    if cfg["mode"] == "mx":
        assert np.array_equal(gs, s), cfg
    else:
        assert np.array_equal(gs.view(np.uint32), s.view(np.uint32)), cfg


def _run_silu(gu, mode):
    qa = afq.silu_mul_quant(dev16(gu), MODE[mode], want_act=True)
    torch.cuda.synchronize()
    return dict(values=host8(qa.values), scales=scales_u8_or_f32(qa.scales), act=host16(qa.normed))


@pytest.mark.parametrize("M", [8, 16, 192, 300])
def test_silu_mx_i768(M):
    gu = inputs.gate_up_inputs(M, 768, seed=0, std=2.0)
    gpu = _run_silu(gu, "mx")
    ref = orc.silu_quant(gu, orc.MXFP8, threads=8)
    n1 = check_codes(gpu["values"], ref["values"], "silu-mx")
    nb, _ = check_scales(gpu["scales"], ref["scales"], 0, "silu-mx")
    na = check_dtype16(gpu["act"], ref["act"], "silu-mx act")
    _report(f"silu-mx M={M}", dict(codes_1=n1, scales_bad=nb, act_1ulp=na))


@pytest.mark.parametrize("I,M", [(12288, 1), (12288, 32), (3072, 64), (2176, 9), (1536, 33)])
def test_silu_b128(I, M):
    gu = inputs.gate_up_inputs(M, I, seed=1, std=1.0)
    gpu = _run_silu(gu, "b128")
    ref = orc.silu_quant(gu, orc.BLOCK128, threads=8)
    # the bf16 activation of this mode is computed exactly: bit-identical
    check_dtype16(gpu["act"], ref["act"], "silu-b128 act", exact=True)
    assert np.array_equal(gpu["values"], ref["values"])
    assert np.array_equal(gpu["scales"].view(np.uint32), ref["scales"].view(np.uint32))


def test_silu_b128_all_gates_exact():
    """bf16(silu(g)) for every finite bf16 gate (up = 1): bit-identical."""
    c = np.arange(1 << 16, dtype=np.uint32)
    gates = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pad = (-gates.size) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    one = inputs.to_bits(np.ones(1))[0]
    gu = np.concatenate([g, np.full_like(g, one)], axis=1)
    gpu = _run_silu(gu, "b128")
    ref = orc.silu_quant(gu, orc.BLOCK128, threads=8)
    bad = np.flatnonzero(gpu["act"].ravel() != ref["act"].ravel())
    assert bad.size == 0, [hex(int(gu.reshape(-1, 256)[i // 128, i % 128])) for i in bad[:10]]
    assert np.array_equal(gpu["values"], ref["values"])


def test_silu_b128_flagged_gates_mixed_in_chunks():
    """Chunks that mix the gates whose fast SiLU sits at a bf16 rounding
    midpoint (5.9375, whose exact value the kernel holds as an immediate,
    and 2^-7, -2^-8, odd subnormals, which it reads from the table), gates
    below -80 (table) and ordinary gates, in every lane position of a chunk:
    the activation bit-identical to the oracle."""
    b = lambda v: int(inputs.to_bits(np.array([v]))[0])
    special = [b(5.9375), b(2.0 ** -7), b(-(2.0 ** -8)), 0x0003, 0x8005, b(-100.0), b(-85.5)]
    rng = np.random.default_rng(17)
    rows = []
    for _ in range(96):
        g = inputs.to_bits(rng.normal(0.0, 3.0, 128))
        for pos in rng.choice(128, size=rng.integers(1, 12), replace=False):
            g[pos] = special[rng.integers(len(special))]
        rows.append(g)
    # and chunks of the midpoint gate alone, and with one other flagged gate
    rows.append(np.full(128, special[0], np.uint16))
    for other in special[1:]:
        for lane in range(8):
            g = np.full(128, special[0], np.uint16)
            g[lane::8] = other
            rows.append(g)
    g = np.stack(rows).astype(np.uint16)
    up = inputs.to_bits(rng.normal(0.0, 1.0, g.shape))
    gu = np.concatenate([g, up], axis=1)
    gpu = _run_silu(gu, "b128")
    ref = orc.silu_quant(gu, orc.BLOCK128, threads=8)
    check_dtype16(gpu["act"], ref["act"], "silu-b128 flagged act", exact=True)
    assert np.array_equal(gpu["values"], ref["values"])
    assert np.array_equal(gpu["scales"].view(np.uint32), ref["scales"].view(np.uint32))


# Launches of at least this many chunks (8 activations each) are the
# bandwidth-bound prefill sizes; their rows must equal the same rows run as
# a small launch (batch invariance) as well as the oracle.
_LARGE_CHUNKS = 1 << 20


def _silu_rows_small(gu, rows, mode):
    """The given rows of gate_up run as their own (small) launch."""
    return _run_silu(np.ascontiguousarray(gu[rows]), mode)


@pytest.mark.parametrize("I,M,seed,std", [(12288, 4096, 0, 1.0),    # benchmark workloads
                                          (3072, 16384, 1, 3.0),
                                          (2176, 3900, 5, 2.0)])     # ragged last step
def test_silu_b128_large_launch_all_rows(I, M, seed, std):
    """The 1x128 SiLU-and-mul at the benchmark sizes (I = 12288, M = 4096;
    I = 3072, M = 16384) and a ragged one: every row bit-exact against the
    oracle, and 48 sampled rows equal to the same rows run as a small launch
    (batch invariance)."""
    assert M * I // 8 >= _LARGE_CHUNKS
    print(f"case silu b128 large I={I} M={M}", flush=True)
    gu = inputs.gate_up_inputs(M, I, seed=seed, std=std)
    qa = afq.silu_mul_quant(dev16(gu), afq.BLOCK128)   # launched as timed: no copy
    torch.cuda.synchronize()
    values, scales = host8(qa.values), scales_u8_or_f32(qa.scales)
    del qa
    ref = orc.silu_quant(gu, orc.BLOCK128, threads=HOST_THREADS, want_act=False)
    bad = np.flatnonzero(values.ravel() != ref["values"].ravel())
    assert bad.size == 0, f"{bad.size} codes differ, first at {bad[:5]}"
    assert np.array_equal(scales.view(np.uint32), ref["scales"].view(np.uint32))
    rows = np.sort(np.random.default_rng(seed).choice(M, 48, replace=False))
    rows[0], rows[-1] = 0, M - 1
    small = _silu_rows_small(gu, rows, "b128")
    assert np.array_equal(values[rows], small["values"])
    assert np.array_equal(scales[rows].view(np.uint32), small["scales"].view(np.uint32))
    ref_rows = orc.silu_quant(gu[rows], orc.BLOCK128)
    check_dtype16(small["act"], ref_rows["act"], "silu-b128 rows act", exact=True)


def test_silu_b128_large_launch_all_gates():
    """Every finite bf16 gate (up = 1), tiled into a prefill-sized launch:
    bit-identical to the oracle in every tile."""
    c = np.arange(1 << 16, dtype=np.uint32)
    gates = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pad = (-gates.size) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    one = inputs.to_bits(np.ones(1))[0]
    block = np.concatenate([g, np.full_like(g, one)], axis=1)
    reps = -(-_LARGE_CHUNKS // (block.shape[0] * 16))
    gu = np.tile(block, (reps, 1))
    assert gu.shape[0] * 16 >= _LARGE_CHUNKS
    gpu = _run_silu(gu, "b128")
    ref = orc.silu_quant(block, orc.BLOCK128, threads=8)
    n = block.shape[0]
    for r in range(reps):
        sl = slice(r * n, (r + 1) * n)
        assert np.array_equal(gpu["act"][sl], ref["act"]), r
        assert np.array_equal(gpu["values"][sl], ref["values"]), r
        assert np.array_equal(gpu["scales"][sl].view(np.uint32), ref["scales"].view(np.uint32)), r


def test_silu_mx_extreme_gates():
    rng = np.random.default_rng(9)
    g = rng.standard_normal((4, 256)) * 30.0
    g[0, :64] = -rng.uniform(80, 100, 64)     # e^-g beyond the fp32 range
    g[1, :] = rng.uniform(-95, -85, 256)       # whole blocks of tiny activations
    u = rng.standard_normal((4, 256)) * 2.0
    gu = np.concatenate([inputs.to_bits(g), inputs.to_bits(u)], axis=1)
    gpu = _run_silu(gu, "mx")
    ref = orc.silu_quant(gu, orc.MXFP8)
    check_codes(gpu["values"], ref["values"], "silu-mx-extreme")
    check_scales(gpu["scales"], ref["scales"], 0, "silu-mx-extreme")


def test_silu_b128_all_gates_many_ups():
    """1x128 SiLU-and-mul for every finite bf16 gate times seven up values
    (-2.75, 2^-10, 3e-3, 96, -2^40, 2^-100, 1e20): the activation
    bit-identical to the oracle (the path's arithmetic is exact: bf16(silu),
    an exact product, one rounding), and the codes and scales of every group
    whose activation stays finite too (an activation that overflows the bf16
    range leaves its group's outputs unspecified)."""
    c = np.arange(1 << 16, dtype=np.uint32)
    gates = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pad = (-gates.size) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    ups = inputs.to_bits(np.array([-2.75, 2.0 ** -10, 3e-3, 96.0, -(2.0 ** 40), 2.0 ** -100, 1e20]))
    gu = np.concatenate([np.concatenate([g, np.full_like(g, u)], axis=1) for u in ups], axis=0)
    gpu = _run_silu(gu, "b128")
    ref = orc.silu_quant(gu, orc.BLOCK128, threads=8)
    bad = np.flatnonzero(gpu["act"].ravel() != ref["act"].ravel())
    assert bad.size == 0, [(hex(int(gu.ravel()[0])), int(i)) for i in bad[:5]]
    # groups whose activation overflows (silu(g) * up beyond the bf16 range)
    # have unspecified codes and scales; every other group is bit-exact
    inf = (ref["act"] & 0x7FFF) == 0x7F80
    ok = ~inf.reshape(gu.shape[0], -1, 128).any(axis=2)          # [rows, groups]
    assert np.array_equal(gpu["scales"].view(np.uint32)[ok], ref["scales"].view(np.uint32)[ok])
    okel = np.repeat(ok, 128, axis=1)
    assert np.array_equal(gpu["values"][okel], ref["values"][okel])
    _report("silu-b128 all gates x 7 ups", dict(groups=int(ok.size), overflowing_groups=int((~ok).sum())))


def test_silu_mx_all_gates():
    """MXFP8 SiLU-and-mul for every finite bf16 gate times eight up values
    across the exponent range (1, -2.75, 2^-10, 3e-3, 96, -2^40, 2^-100,
    1e30): the bf16 copy of the fp32 activation within 1 ulp of the oracle's
    (the kernel's silu is within 2 fp32 ulp), codes and scales within the
    budget, and the codes equal to the oracle quantiser applied to the
    kernel's own activation."""
    c = np.arange(1 << 16, dtype=np.uint32)
    gates = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pad = (-gates.size) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    ups = inputs.to_bits(np.array([1.0, -2.75, 2.0 ** -10, 3e-3, 96.0, -(2.0 ** 40), 2.0 ** -100, 1e30]))
    gu = np.concatenate([np.concatenate([g, np.full_like(g, u)], axis=1) for u in ups], axis=0)
    gpu = _run_silu(gu, "mx")
    ref = orc.silu_quant(gu, orc.MXFP8, threads=8)
    n_act = check_dtype16(gpu["act"], ref["act"], "silu-mx all gates act")
    n_codes = check_codes(gpu["values"], ref["values"], "silu-mx all gates")
    n_sc, _ = check_scales(gpu["scales"], ref["scales"], 0, "silu-mx all gates")
    _report("silu-mx all gates x 8 ups", dict(elements=int(gu.shape[0] * 128), act_1ulp=n_act,
                                               codes_1=n_codes, scales_bad=n_sc))


# --------------------------------------------------------- standalone quant
@pytest.mark.parametrize("dtype", ["bf16", "fp16", "fp32"])
@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
def test_fp8_quant_standalone(dtype, mode):
    rng = np.random.default_rng(10)
    M, n = 37, 3072
    x = rng.standard_normal((M, n)) * 2.0 ** rng.integers(-12, 12, (M, 1))
    x[0] = 0.0
    x[1, ::5] *= 1000.0
    if dtype == "fp32":
        xh = x.astype(np.float32)
        xt = torch.from_numpy(xh).cuda()
        odt = orc.FP32
    else:
        xh = inputs.to_bits(x, dtype)
        xt = dev16(xh, dtype)
        odt = ORC_DT[dtype]
    qa = afq.fp8_quant(xt, MODE[mode])
    torch.cuda.synchronize()
    q, s = orc.quant(xh, odt, MODE[mode], threads=8)
    assert np.array_equal(host8(qa.values), q)
    gs = scales_u8_or_f32(qa.scales)
    if mode == "mx":
        assert np.array_equal(gs, s)
    else:
        assert np.array_equal(gs.view(np.uint32), s.view(np.uint32))


def test_fp8_quant_mx_every_bf16_value_under_every_block_exponent():
    """The MXFP8 quantiser kernel over every finite bf16 value u under every
    block exponent that admits it (blocks of 32: the largest bf16 of fp32
    exponent field E, then values of field <= E; E = 1..254; 8.3 M
    elements): scale bytes and codes bit-identical to the oracle."""
    c = np.arange(1 << 16, dtype=np.uint32)
    fin = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    field = (fin.astype(np.uint32) >> 7) & 0xFF
    blocks = []
    for E in range(1, 255):
        vals = fin[field <= E]
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blocks.append(np.concatenate([np.full((n, 1), np.uint16((E << 7) | 0x7F), np.uint16),
                                      pad.reshape(n, 31)], axis=1))
    x = np.concatenate(blocks)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 192, 32), np.uint16)]).reshape(-1, 6144)
    qa = afq.fp8_quant(dev16(x), afq.MXFP8)
    torch.cuda.synchronize()
    q, sc = orc.quant(x, orc.BF16, orc.MXFP8, threads=8)
    assert np.array_equal(scales_u8_or_f32(qa.scales), sc)
    bad = np.argwhere(host8(qa.values) != q)
    assert bad.size == 0, [(int(x[tuple(b)]), int(host8(qa.values)[tuple(b)]), int(q[tuple(b)])) for b in bad[:5]]


def test_fp8_quant_mx_every_fp16_value_under_every_block_exponent():
    """The same sweep for fp16 input: every finite fp16 value u under every
    block exponent that admits it (fp16 subnormals are normal in fp32, so
    the block exponents are taken from the fp32 exponent field of the
    decoded values), bit-identical to the oracle."""
    c = np.arange(1 << 16, dtype=np.uint32)
    fin = c[((c >> 10) & 0x1F) != 0x1F].astype(np.uint16)
    val = fin.view(np.float16).astype(np.float32)
    field = (val.view(np.uint32) >> 23) & 0xFF                  # 0 only for +-0
    pos = fin[(fin & 0x8000) == 0]
    pos_field = (pos.view(np.float16).astype(np.float32).view(np.uint32) >> 23) & 0xFF
    blocks = []
    for E in np.unique(pos_field[pos_field > 0]):
        amax = pos[pos_field == E].max()                         # largest fp16 of this exponent
        vals = fin[field <= E]
        n = -(-vals.size // 31)
        pad = np.zeros(n * 31, np.uint16)
        pad[:vals.size] = vals
        blocks.append(np.concatenate([np.full((n, 1), amax, np.uint16), pad.reshape(n, 31)], axis=1))
    x = np.concatenate(blocks)
    x = np.concatenate([x, np.zeros(((-x.shape[0]) % 192, 32), np.uint16)]).reshape(-1, 6144)
    qa = afq.fp8_quant(dev16(x, "fp16"), afq.MXFP8)
    torch.cuda.synchronize()
    q, sc = orc.quant(x, orc.FP16, orc.MXFP8, threads=8)
    assert np.array_equal(scales_u8_or_f32(qa.scales), sc)
    assert np.array_equal(host8(qa.values), q)
    _report("mx quant every fp16 value", dict(elements=int(x.size), block_exponents=len(blocks)))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
@pytest.mark.parametrize("n", [256, 3072, 8192, 20480, 32768])
def test_fp8_quant_per_token_bandwidth_shapes(dtype, n):
    """The standalone per-token quantiser at 1100 rows, where its row shape
    takes one chunk per lane at width 256 (64 lanes, four rows per block),
    two at 3072, three at 8192 and 20480 (a round at two holds fewer rows)
    and four at 32768: bit-exact."""
    rng = np.random.default_rng(11)
    M = 1100
    x = rng.standard_normal((M, n)) * 2.0 ** rng.integers(-8, 8, (M, 1))
    if dtype == "fp32":
        xh = x.astype(np.float32)
        xt = torch.from_numpy(xh).cuda()
        odt = orc.FP32
    else:
        xh = inputs.to_bits(x, dtype)
        xt = dev16(xh, dtype)
        odt = ORC_DT[dtype]
    qa = afq.fp8_quant(xt, afq.PER_TOKEN)
    torch.cuda.synchronize()
    q, s = orc.quant(xh, odt, afq.PER_TOKEN, threads=8)
    assert np.array_equal(host8(qa.values), q)
    assert np.array_equal(scales_u8_or_f32(qa.scales).view(np.uint32), s.view(np.uint32))


@pytest.mark.parametrize("dtype,n,M", [
    ("bf16", 256, 7),      # one chunk per lane, 64 lanes, four rows per block (a ragged block)
    ("bf16", 8192, 300),   # two chunks per lane
    ("fp16", 8192, 1100),  # three
    ("fp32", 8192, 1100),  # three, fp32 input (two loads per chunk)
    ("bf16", 32768, 5),    # four
])
def test_fp8_quant_per_token_strided_rows(dtype, n, M):
    """The per-token quantiser on a column slice of a wider buffer (row
    stride above the row): every lane loads without a branch, lanes past
    the row or past the last row from an in-bounds chunk of the last row,
    so the row stride enters every address.  Bit-exact against the oracle
    on the slice's contiguous copy."""
    print(f"case strided per-token quant {dtype} n={n} M={M}", flush=True)
    rng = np.random.default_rng(29)
    x = rng.standard_normal((M, n + 64)) * 2.0 ** rng.integers(-8, 8, (M, 1))
    x[:, 16 + n:] = 1e30 if dtype == "fp32" else 6e4  # past the slice: must not enter any max
    if dtype == "fp32":
        xh = x.astype(np.float32)
        xt = torch.from_numpy(xh).cuda()
        odt = orc.FP32
    else:
        xh = inputs.to_bits(x, dtype)
        xt = dev16(xh, dtype)
        odt = ORC_DT[dtype]
    qa = afq.fp8_quant(xt[:, 16:16 + n], afq.PER_TOKEN)
    torch.cuda.synchronize()
    q, sc = orc.quant(np.ascontiguousarray(xh[:, 16:16 + n]), odt, afq.PER_TOKEN, threads=8)
    assert np.array_equal(host8(qa.values), q)
    assert np.array_equal(scales_u8_or_f32(qa.scales).view(np.uint32), sc.view(np.uint32))


def test_fp8_quant_per_token_rows_independent_of_shape():
    """The standalone per-token quantiser's row shape follows the row count
    (width 8192: two chunks per lane up to 1024 rows, three above): the
    first 8 rows come out bit-identical from every launch, and equal to the
    oracle's."""
    rng = np.random.default_rng(23)
    n = 8192
    xh = inputs.to_bits(rng.standard_normal((2048, n)) * 2.0 ** rng.integers(-8, 8, (2048, 1)), "bf16")
    xt = dev16(xh, "bf16")
    q, s = orc.quant(xh[:8], ORC_DT["bf16"], afq.PER_TOKEN, threads=8)
    for M in (8, 300, 1100, 2048):
        print(f"case per-token quant shape M={M}", flush=True)
        qa = afq.fp8_quant(xt[:M], afq.PER_TOKEN)
        torch.cuda.synchronize()
        assert np.array_equal(host8(qa.values)[:8], q), M
        assert np.array_equal(scales_u8_or_f32(qa.scales)[:8].view(np.uint32), s.view(np.uint32)), M


@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_fused_norm_equals_norm_then_quant(mode, dtype):
    """Fused = unfused on the GPU: the fused codes and scales equal the
    standalone quantiser applied to the fused kernel's own normed copy (the
    quantiser's input is the dtype-rounded norm output in every mode)."""
    M, H = 300, 6144
    d = inputs.norm_inputs(M, H, seed=11, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1,
                           dtype=dtype)
    qa = afq.fused_add_rmsnorm_quant(dev16(d["x"], dtype), dev16(d["w"], dtype), 1e-6,
                                     mode=MODE[mode], kind=afq.GEMMA, residual=dev16(d["r"], dtype),
                                     want_normed=True)
    sep = afq.fp8_quant(qa.normed, MODE[mode])
    torch.cuda.synchronize()
    assert np.array_equal(host8(qa.values), host8(sep.values))
    assert np.array_equal(scales_u8_or_f32(qa.scales).view(np.uint8),
                          scales_u8_or_f32(sep.scales).view(np.uint8))


def test_fused_silu_b128_equals_silu_then_quant():
    """1x128 SiLU-and-mul quantises the bf16 activation it returns: the codes
    equal the standalone 1x128 quantiser applied to that activation."""
    gu = inputs.gate_up_inputs(257, 3072, seed=12, std=3.0)
    qa = afq.silu_mul_quant(dev16(gu), afq.BLOCK128, want_act=True)
    sep = afq.fp8_quant(qa.normed, afq.BLOCK128)
    torch.cuda.synchronize()
    assert np.array_equal(host8(qa.values), host8(sep.values))
    assert np.array_equal(scales_u8_or_f32(qa.scales).view(np.uint32),
                          scales_u8_or_f32(sep.scales).view(np.uint32))


@pytest.mark.parametrize("mode", ["mx", "b128", "pt"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_unfused_norm_chain_equals_fused(mode, dtype):
    """The unfused chain on this library's kernels -- a copy-only norm launch,
    then fp8_quant of its rows -- equals the fused launch bit for bit:
    residual, normed rows, codes and scales ([P1] "Test Plan /
    Correctness" states this of the fused MXFP8 norm)."""
    M, H = 37, 6144
    d = inputs.norm_inputs(M, H, seed=31, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1,
                           dtype=dtype)
    x, w, r = dev16(d["x"], dtype), dev16(d["w"], dtype), dev16(d["r"], dtype)
    fused = afq.fused_add_rmsnorm_quant(x, w, 1e-6, mode=MODE[mode], kind=afq.GEMMA, residual=r,
                                        want_normed=True)
    plain = afq.fused_add_rmsnorm_quant(x, w, 1e-6, mode=MODE[mode], kind=afq.GEMMA, residual=r,
                                        quantize=False)
    assert plain.values is None and plain.scales is None
    q = afq.fp8_quant(plain.normed, MODE[mode])
    torch.cuda.synchronize()
    assert torch.equal(plain.residual, fused.residual)
    assert torch.equal(plain.normed.view(torch.int16), fused.normed.view(torch.int16))
    assert torch.equal(q.values.view(torch.uint8), fused.values.view(torch.uint8))
    assert torch.equal(q.scales.view(torch.uint8), fused.scales.view(torch.uint8))
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode=mode, dtype=dtype)
    check_dtype16(host16(plain.normed), ref["normed"], f"copy-only {mode} {dtype}")


def test_copy_only_norm_odd_width_and_two_segments():
    """A copy-only launch needs no quantisation groups (width 200 = 25
    chunks), and a two-segment copy-only launch writes both segments' rows."""
    d = inputs.norm_inputs(11, 200, seed=33, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    plain = afq.fused_add_rmsnorm_quant(dev16(d["x"]), dev16(d["w"]), 1e-6, mode=afq.PER_TOKEN,
                                        kind=afq.STANDARD, residual=dev16(d["r"]), quantize=False)
    torch.cuda.synchronize()
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="pt")
    check_dtype16(host16(plain.residual), ref["h"], "copy-only w200 h", exact=True)
    check_dtype16(host16(plain.normed), ref["normed"], "copy-only w200")
    segs = inputs.two_segment_inputs(9, (1536, 512), seed=34)
    xs = [dev16(sg["x"]) for sg in segs]
    ws = [dev16(sg["w"]) for sg in segs]
    fused = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=afq.PER_TOKEN, kind=afq.STANDARD,
                                        want_normed=True)
    plain = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=afq.PER_TOKEN, kind=afq.STANDARD,
                                        quantize=False)
    torch.cuda.synchronize()
    for f, p in zip(fused, plain):
        assert p.values is None and torch.equal(p.normed.view(torch.int16), f.normed.view(torch.int16))


@pytest.mark.parametrize("mode,I", [("mx", 768), ("b128", 3072)])
def test_unfused_silu_chain(mode, I):
    """The unfused SiLU chain on this library's kernels -- a copy-only
    SiLU-and-mul launch, then fp8_quant of its bf16 activation.  1x128: equal
    to the fused launch bit for bit ([P2] "Modifications").  MXFP8: equal to
    the fused bf16-first variant bit for bit; the default MXFP8 fusion
    quantises the fp32 activation instead, so a few % of its codes differ
    ([P1] "Test Plan / Correctness")."""
    gu = inputs.gate_up_inputs(29, I, seed=32, std=2.0)
    g = dev16(gu)
    fused = afq.silu_mul_quant(g, MODE[mode], want_act=True)
    plain = afq.silu_mul_quant(g, MODE[mode], quantize=False)
    assert plain.values is None and plain.scales is None
    q = afq.fp8_quant(plain.normed, MODE[mode])
    torch.cuda.synchronize()
    assert torch.equal(plain.normed.view(torch.int16), fused.normed.view(torch.int16))
    ref = orc.silu_quant(gu, MODE[mode], threads=8)
    check_dtype16(host16(plain.normed), ref["act"], f"copy-only silu {mode}", exact=(mode == "b128"))
    if mode == "b128":
        assert torch.equal(q.values.view(torch.uint8), fused.values.view(torch.uint8))
        assert torch.equal(q.scales.view(torch.uint8), fused.scales.view(torch.uint8))
    else:
        bf = afq.silu_mul_quant(g, afq.MXFP8, quant_input=afq.QIN_BF16)
        torch.cuda.synchronize()
        assert torch.equal(q.values.view(torch.uint8), bf.values.view(torch.uint8))
        assert torch.equal(q.scales, bf.scales)
        differ = (q.values.view(torch.uint8) != fused.values.view(torch.uint8)).float().mean().item()
        _report(f"silu mx: unfused chain vs fp32 fusion", dict(codes_differ=round(differ, 4)))
        assert differ < 0.1


def test_e4m3_conversion_structured_fp32():
    """Every fp32 exponent that reaches e4m3 (codes 0..448), all 2^5 top
    mantissa patterns times boundary low bits, both signs: quantised with
    unit scale (each 32-block holds a 256.0 anchor, so the E8M0 byte is
    127) and compared code by code with the oracle."""
    exps = np.arange(0, 136, dtype=np.uint32)          # up to 2^8 binade
    top = np.arange(32, dtype=np.uint32) << 18
    low = np.array([0, 1, 2, 0x1FFFF, 0x20000, 0x20001, 0x3FFFF, 0x10000, 0x30000], dtype=np.uint32)
    bits = (exps[:, None, None] << 23) | top[None, :, None] | low[None, None, :]
    bits = bits.ravel()
    bits = np.concatenate([bits, bits | np.uint32(0x80000000)])
    vals = bits.view(np.float32)
    vals = vals[np.abs(vals) <= 448]
    per = 31
    nblk = (vals.size + per - 1) // per
    buf = np.zeros((nblk, 32), np.float32)
    flat = np.zeros(nblk * per, np.float32)
    flat[:vals.size] = vals
    buf[:, 1:] = flat.reshape(nblk, per)
    buf[:, 0] = 256.0
    cols = 32 * 64
    pad = (-nblk) % 64
    buf = np.concatenate([buf, np.zeros((pad, 32), np.float32)]).reshape(-1, cols)
    qa = afq.fp8_quant(torch.from_numpy(buf).cuda(), afq.MXFP8)
    torch.cuda.synchronize()
    q, s = orc.quant(buf, orc.FP32, orc.MXFP8, threads=8)
    got = host8(qa.values)
    bad = np.flatnonzero(got.ravel() != q.ravel())
    assert bad.size == 0, [(float(buf.ravel()[i]), hex(got.ravel()[i]), hex(q.ravel()[i])) for i in bad[:8]]


def test_fp32_quotient_exact_bf16_all_values():
    """1x128 codes of every positive bf16 mantissa against group maxima of
    every mantissa: e4m3(fp32(u/s)) must match the oracle exactly."""
    rng = np.random.default_rng(11)
    mant = np.arange(128)
    rows = []
    for am in range(128):
        A = (1 + am / 128.0) * 2.0 ** int(rng.integers(-20, 20))
        # 127 values in [0, A] drawn from all mantissas / nearby exponents, then the max
        e = np.floor(np.log2(A))
        v = (1 + rng.permutation(mant)[:127] / 128.0) * 2.0 ** (e - rng.integers(0, 12, 127))
        v = np.minimum(v, A) * np.where(rng.random(127) < 0.5, -1, 1)
        rows.append(np.concatenate([[A], v]))
    x = inputs.to_bits(np.array(rows))
    qa = afq.fp8_quant(dev16(x), afq.BLOCK128)
    torch.cuda.synchronize()
    q, s = orc.quant(x, orc.BF16, orc.BLOCK128)
    assert np.array_equal(host8(qa.values), q)


# ------------------------------------------------------ execution properties
def test_deterministic_and_batch_invariant():
    d = inputs.norm_inputs(67, 6144, seed=12, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    a = run_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode="mx")
    b = run_norm(d["x"], d["w"], r=d["r"], kind="gemma", mode="mx")
    for k in ("h", "normed", "values", "scales"):
        assert np.array_equal(a[k], b[k]), k
    c = run_norm(d["x"][5:13], d["w"], r=d["r"][5:13], kind="gemma", mode="mx")
    for k in ("h", "normed", "values", "scales"):
        assert np.array_equal(a[k][5:13], c[k]), k


def test_bitwise_determinism_many_runs():
    """50 launches of each path (one and two LDS barriers, fp64 reduction,
    flat SiLU) into fresh outputs, each bit for bit equal to the first: the
    reductions have a fixed order and no launch depends on another."""
    d = inputs.norm_inputs(67, 6144, seed=17, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    xt, wt, rt = dev16(d["x"]), dev16(d["w"]), dev16(d["r"])
    segs = inputs.two_segment_inputs(300, (1536, 512), seed=18)
    xs = [dev16(sg["x"]) for sg in segs]
    ws = [dev16(sg["w"]) for sg in segs]
    gu = dev16(inputs.gate_up_inputs(64, 3072, seed=19, std=2.0))
    d4 = inputs.norm_inputs(40, 4096, seed=20, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    x4, w4, r4 = dev16(d4["x"]), dev16(d4["w"]), dev16(d4["r"])

    def once():
        a = afq.fused_add_rmsnorm_quant(xt, wt, 1e-6, mode=afq.MXFP8, kind=afq.GEMMA, residual=rt,
                                        want_normed=True)
        b = afq.fused_add_rmsnorm_quant(xs, ws, 1e-6, mode=afq.PER_TOKEN, kind=afq.STANDARD)
        c = afq.silu_mul_quant(gu, afq.BLOCK128, want_act=True)
        e = afq.fused_add_rmsnorm_quant(x4, w4, 1e-6, mode=afq.BLOCK128, kind=afq.STANDARD,
                                        residual=r4, quant_input=afq.QIN_FP32)
        outs = [a.values, a.scales, a.normed, a.residual, b[0].values, b[0].scales, b[1].values,
                b[1].scales, c.values, c.scales, c.normed, e.values, e.scales, e.residual]
        return [t.view(torch.uint8) if t.dtype != torch.float32 else t.view(torch.int32) for t in outs]

    first = [t.clone() for t in once()]
    for _ in range(49):
        for t0, t in zip(first, once()):
            assert torch.equal(t0, t)
    torch.cuda.synchronize()


GRAPH_ROW_COUNTS = list(range(1, 65)) + list(range(72, 513, 8))


@pytest.mark.parametrize("mode,kind", [("mx", "gemma"), ("b128", "standard"), ("pt", "standard")])
def test_norm_every_graph_row_count(mode, kind):
    """Every row count 1..64 and every graph-capture size up to 512 (steps of
    8), at hidden 2048: each launch on the first M rows of one 512-row input
    matches the oracle's first M rows (rows are independent, so this is also
    batch invariance), and row 0 is bit-identical across all M."""
    d = inputs.norm_inputs(512, 2048, seed=21, x_std=3.0, r_std=1.0,
                           w_kind="normal" if kind == "gemma" else "uniform",
                           w_param=0.1 if kind == "gemma" else 0.5)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode)
    first = None
    for M in GRAPH_ROW_COUNTS:
        gpu = run_norm(d["x"][:M], d["w"], r=d["r"][:M], kind=kind, mode=mode)
        sub = {k: ref[k][:M] for k in ("h", "normed", "values", "scales")}
        check_norm(gpu, sub, mode, "bf16", f"rows{M}-{mode}")
        row0 = (gpu["values"][0].tobytes(), np.ascontiguousarray(gpu["scales"][0]).tobytes(),
                gpu["normed"][0].tobytes())
        first = first or row0
        assert row0 == first, f"row 0 differs at M={M}"


@pytest.mark.parametrize("mode,I", [("mx", 768), ("b128", 2176)])
def test_silu_every_graph_row_count(mode, I):
    """SiLU-and-mul at every row count 1..64 and every graph size up to 512,
    on prefixes of one 512-row input, against the oracle's rows."""
    gu = inputs.gate_up_inputs(512, I, seed=22, std=2.0)
    ref = orc.silu_quant(gu, MODE[mode], threads=8)
    for M in GRAPH_ROW_COUNTS:
        gpu = _run_silu(gu[:M], mode)
        if mode == "b128":
            assert np.array_equal(gpu["values"], ref["values"][:M]), M
            assert np.array_equal(gpu["scales"].view(np.uint32), ref["scales"][:M].view(np.uint32)), M
        else:
            check_codes(gpu["values"], ref["values"][:M], f"silu-mx rows{M}")
            check_scales(gpu["scales"], ref["scales"][:M], 0, f"silu-mx rows{M}")
            check_dtype16(gpu["act"], ref["act"][:M], f"silu-mx rows{M} act")


def test_graph_replay_equals_eager():
    d = inputs.norm_inputs(32, 6144, seed=13, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    xt, wt, rt = dev16(d["x"]), dev16(d["w"]), dev16(d["r"])
    eager = afq.fused_add_rmsnorm_quant(xt, wt, 1e-6, mode=afq.MXFP8, kind=afq.GEMMA, residual=rt,
                                        want_normed=True)
    gu = dev16(inputs.gate_up_inputs(32, 768, seed=13, std=2.0))
    eager_s = afq.silu_mul_quant(gu, afq.MXFP8)
    torch.cuda.synchronize()
    outs = (torch.empty_like(eager.values), torch.empty_like(eager.scales), torch.empty_like(eager.normed))
    res_out = torch.empty_like(rt)
    souts = (torch.empty_like(eager_s.values), torch.empty_like(eager_s.scales), None)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            afq.fused_add_rmsnorm_quant(xt, wt, 1e-6, mode=afq.MXFP8, kind=afq.GEMMA, residual=rt,
                                        residual_out=res_out, want_normed=True, out=outs)
            afq.silu_mul_quant(gu, afq.MXFP8, out=souts)
    torch.cuda.current_stream().wait_stream(s)
    for rep in range(3):
        for t in (*outs, res_out, souts[0], souts[1]):
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        assert torch.equal(outs[0].view(torch.uint8), eager.values.view(torch.uint8)), rep
        assert torch.equal(outs[1], eager.scales), rep
        assert torch.equal(outs[2], eager.normed), rep
        assert torch.equal(res_out, eager.residual), rep
        assert torch.equal(souts[0].view(torch.uint8), eager_s.values.view(torch.uint8)), rep
        assert torch.equal(souts[1], eager_s.scales), rep


def test_guard_bands_untouched():
    """Outputs carved from larger poisoned buffers: bytes outside each output
    stay untouched, bytes inside are all written."""
    M, H = 9, 2048
    d = inputs.norm_inputs(M, H, seed=14, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    for mode in ("mx", "b128", "pt"):
        sshape = {"mx": (M, H // 32), "b128": (M, H // 128), "pt": (M, 1)}[mode]
        sbytes = int(np.prod(sshape)) * (1 if mode == "mx" else 4)
        guard = 256
        vb = torch.full((M * H + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
        sb = torch.full((sbytes + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
        nb = torch.full((M * H * 2 + 2 * guard,), 0x5A, dtype=torch.uint8, device="cuda")
        values = vb[guard:guard + M * H].view(torch.float8_e4m3fn).view(M, H)
        scales = sb[guard:guard + sbytes]
        scales = scales.view(sshape) if mode == "mx" else scales.view(torch.float32).view(sshape)
        normed = nb[guard:guard + 2 * M * H].view(torch.bfloat16).view(M, H)
        afq.fused_add_rmsnorm_quant(dev16(d["x"]), dev16(d["w"]), 1e-6, mode=MODE[mode],
                                    kind=afq.STANDARD, residual=dev16(d["r"]),
                                    out=(values, scales, normed))
        torch.cuda.synchronize()
        for buf in (vb, sb, nb):
            assert bool((buf[:guard] == 0x5A).all()) and bool((buf[-guard:] == 0x5A).all()), mode
        ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode=mode)
        check_codes(host8(values), ref["values"], mode)
        check_scales(scales_u8_or_f32(scales), ref["scales"], MODE[mode], mode, u=ref["normed"],
                     dtype="bf16")
        check_dtype16(host16(normed), ref["normed"], mode)


def test_rejected_call_writes_nothing():
    M, H = 4, 256
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    values = torch.full((M, H), 7, dtype=torch.uint8, device="cuda").view(torch.float8_e4m3fn)
    scales = torch.full((M, H // 32), 9, dtype=torch.uint8, device="cuda")
    with pytest.raises(afq.AfqError) as e:
        # scales overlapping the codes: an alias error, detected by the library
        overlapping = values.view(torch.uint8).view(-1)[: M * (H // 32)].view(M, H // 32)
        afq.fused_add_rmsnorm_quant(x, w, 1e-6, mode=afq.MXFP8, out=(values, overlapping, None))
    assert e.value.status == -5
    torch.cuda.synchronize()
    assert bool((values.view(torch.uint8) == 7).all())


def test_binding_rejects_bad_buffers():
    """Tensors that the kernels would read from host memory or write out of
    bounds are rejected by the Python binding before any launch (the C ABI
    takes raw pointers and cannot see extents or devices)."""
    M, H = 4, 256
    x = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    r = torch.zeros_like(x)
    w = torch.ones(H, dtype=torch.bfloat16, device="cuda")
    vals = torch.full((M, H), 7, dtype=torch.uint8, device="cuda")
    sc = torch.full((M, H // 32), 9, dtype=torch.uint8, device="cuda")
    nrm = torch.zeros((M, H), dtype=torch.bfloat16, device="cuda")
    norm = lambda **k: afq.fused_add_rmsnorm_quant(x if "x" not in k else k.pop("x"),
                                                   w if "w" not in k else k.pop("w"), 1e-6,
                                                   mode=afq.MXFP8, **k)
    bad = [
        ("host weight", lambda: norm(w=w.cpu())),
        ("host residual", lambda: norm(residual=r.cpu())),
        ("short values", lambda: norm(out=(vals[: M - 1], sc, None))),
        ("strided values", lambda: norm(out=(vals.view(H, M).t(), sc, None))),
        ("fp32 MX scales", lambda: norm(out=(vals, sc.view(torch.float32)[:, :2].contiguous(), None))),
        ("short scales", lambda: norm(out=(vals, sc[:, :4].contiguous(), None))),
        ("fp16 copy of bf16 rows", lambda: norm(out=(vals, sc, nrm.view(torch.float16)))),
        ("host values", lambda: norm(out=(vals.cpu(), sc, None))),
        ("short residual_out", lambda: norm(residual=r, residual_out=r[: M - 1])),
        ("fp16 residual_out", lambda: norm(residual=r, residual_out=r.view(torch.float16))),
        ("residual_out alone", lambda: norm(residual_out=r)),
        ("silu short values", lambda: afq.silu_mul_quant(torch.zeros((M, 2 * H), dtype=torch.bfloat16, device="cuda"),
                                                         afq.MXFP8, out=(vals[:, : H // 2], sc, None))),
        ("quant with a copy buffer", lambda: afq.fp8_quant(x, afq.MXFP8, out=(vals, sc, nrm))),
    ]
    for name, call in bad:
        with pytest.raises(ValueError):
            call()
            pytest.fail(name)
    torch.cuda.synchronize()
    assert bool((vals == 7).all()) and bool((sc == 9).all())


# ------------------------------------------------- rounding-point variants
@pytest.mark.parametrize("mode", ["b128", "pt"])
@pytest.mark.parametrize("kind", ["gemma", "standard"])
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("H,M", [(4096, 33), (2048, 5), (6144, 1100)])
def test_norm_fp32_direct(mode, kind, dtype, H, M):
    """fp32-direct: the quantiser reads the fp32 normed value.  The kernel
    takes inv from an fp64 sum of squares rounded once to fp32, as the
    oracle does, and forms the normed value, the scale and the quotient in
    the oracle's fp32 operations: codes, scales and the copy bit-exact."""
    d = inputs.norm_inputs(M, H, seed=15, x_std=2.0, r_std=1.0,
                           w_kind="uniform" if kind == "standard" else "normal",
                           w_param=0.5 if kind == "standard" else 0.1, dtype=dtype)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode, dtype=dtype, qin=afq.QIN_FP32)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode, dtype=dtype, qin=orc.QIN_FP32)
    _report(f"fp32-direct {mode}-{kind}-{dtype} H={H} M={M}",
            check_norm(gpu, ref, mode, dtype, "fp32-direct", requant=False, qin=afq.QIN_FP32))


def test_norm_fp32_direct_edge_rows_and_two_segments():
    """fp32-direct on the edge rows and on the two-segment launch (2048
    rows, the bandwidth row shape): bit-exact."""
    H = 2048
    rows = inputs.edge_rows(H)
    x = inputs.to_bits(rows)
    w = inputs.to_bits(np.random.default_rng(3).uniform(0.5, 1.5, H))
    for mode in ("b128", "pt"):
        gpu = run_norm(x, w, kind="standard", mode=mode, qin=afq.QIN_FP32)
        ref = ref_norm(x, w, kind="standard", mode=mode, qin=orc.QIN_FP32)
        check_norm(gpu, ref, mode, "bf16", f"fp32-direct edge {mode}", requant=False, qin=afq.QIN_FP32)
    M = 2048
    segs = inputs.two_segment_inputs(M, (1536, 512), seed=4)
    buf = np.zeros((M, 2112), np.uint16)
    buf[:, :1536], buf[:, 1536:2048] = segs[0]["x"], segs[1]["x"]
    bt = dev16(buf)
    outs = afq.fused_add_rmsnorm_quant([bt[:, :1536], bt[:, 1536:2048]],
                                       [dev16(segs[0]["w"]), dev16(segs[1]["w"])], 1e-6,
                                       mode=afq.PER_TOKEN, kind=afq.STANDARD, want_normed=True,
                                       quant_input=afq.QIN_FP32)
    torch.cuda.synchronize()
    for sg, qa in zip(segs, outs):
        gpu = dict(normed=host16(qa.normed), values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))
        ref = ref_norm(sg["x"], sg["w"], kind="standard", mode="pt", qin=orc.QIN_FP32)
        _report(f"fp32-direct two-seg cols={sg['x'].shape[1]}",
                check_norm(gpu, ref, "pt", "bf16", "fp32-direct two-seg", requant=False,
                           qin=afq.QIN_FP32))


def test_norm_fp32_direct_prefill_all_rows():
    """The 1x128 fp32-direct launch at the benchmark shape (H = 4096,
    M = 4096), launched as timed; every row against the oracle, bit-exact."""
    M, H = 4096, 4096
    print(f"case fp32-direct prefill M={M} H={H}", flush=True)
    d = inputs.norm_inputs(M, H, seed=0, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="b128", qin=afq.QIN_FP32,
                   want_normed=False)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind="standard", mode="b128", qin=orc.QIN_FP32)
    _report("fp32-direct prefill all rows",
            check_norm(gpu, ref, "b128", "bf16", "fp32-direct prefill", requant=False,
                       qin=afq.QIN_FP32))


@pytest.mark.parametrize("M,I", [(8, 768), (192, 768), (64, 12288), (3, 2176)])
def test_silu_mx_bf16_first(M, I):
    """bf16-first MXFP8 SiLU-and-mul: the quantiser reads the bf16-rounded
    activation.  Against the oracle within the contract, and bit for bit the
    standalone MXFP8 quantiser applied to the kernel's own bf16 activation
    (fused = unfused)."""
    gu = inputs.gate_up_inputs(M, I, seed=5, std=2.0)
    qa = afq.silu_mul_quant(dev16(gu), afq.MXFP8, want_act=True, quant_input=afq.QIN_BF16)
    sep = afq.fp8_quant(qa.normed, afq.MXFP8)
    torch.cuda.synchronize()
    act, values, scales = host16(qa.normed), host8(qa.values), scales_u8_or_f32(qa.scales)
    ref = orc.silu_quant(gu, orc.MXFP8, threads=8, qin=orc.QIN_BF16)
    na = check_dtype16(act, ref["act"], "bf16-first act")
    n1 = check_codes(values, ref["values"], "bf16-first codes")
    nb, _ = check_scales(scales, ref["scales"], 0, "bf16-first scales")
    assert np.array_equal(values, host8(sep.values))
    assert np.array_equal(scales, scales_u8_or_f32(sep.scales))
    _report(f"silu-mx bf16-first M={M} I={I}", dict(act_1ulp=na, codes_1=n1, scales_bad=nb))


# ------------------------------------------------------ split launches
def test_row_kernels_split_large_launches():
    """A row-kernel launch stays below 2^31 work-items: 8-column per-token
    rows take 64 lanes each, so more than 2^25 rows take two launches.  Rows
    on both sides of the split, against the oracle, for the fused norm and
    the standalone per-token quantiser."""
    M, H = (1 << 25) + 1000, 8
    base = inputs.norm_inputs(4096, H, seed=16, x_std=1.0, r_std=None, w_kind="uniform", w_param=0.5)
    x = np.tile(base["x"], (M // 4096 + 1, 1))[:M]
    xt = dev16(x)
    qa = afq.fused_add_rmsnorm_quant(xt, dev16(base["w"]), 1e-6, mode=afq.PER_TOKEN,
                                     kind=afq.STANDARD)
    sep = afq.fp8_quant(xt, afq.PER_TOKEN)
    torch.cuda.synchronize()
    edge = [0, 1, (1 << 25) - 2, (1 << 25) - 1, 1 << 25, (1 << 25) + 1, M - 2, M - 1]
    rows = np.unique(np.concatenate([edge, np.random.default_rng(3).choice(M, 56, replace=False)]))
    idx = torch.from_numpy(rows).cuda()
    pick8 = lambda t: t.view(torch.uint8)[idx].cpu().numpy()
    pickf = lambda t: t[idx].cpu().numpy()
    ref = orc.norm_quant(x[rows], base["w"], kind=orc.STANDARD, dtype=orc.BF16, mode=orc.PER_TOKEN,
                         eps=1e-6)
    check_codes(pick8(qa.values), ref["values"], "split norm codes")
    check_scales(pickf(qa.scales), ref["scales"], 2, "split norm scales", u=ref["normed"], dtype="bf16")
    q, s = orc.quant(x[rows], orc.BF16, orc.PER_TOKEN)
    assert np.array_equal(pick8(sep.values), q)
    assert np.array_equal(pickf(sep.scales).view(np.uint32), s.view(np.uint32))
    del xt, qa, sep
    torch.cuda.empty_cache()


def _split_rows(M, step, base_rows, seed):
    """Rows on both sides of each launch boundary (multiples of `step`),
    the ends, and random rows; with their rows in the tiled base block."""
    edge = [0, 1, M - 2, M - 1]
    for b in range(step, M, step):
        edge += [b - 2, b - 1, b, b + 1]
    rows = np.unique(np.concatenate([edge, np.random.default_rng(seed).choice(M, 40, replace=False)]))
    return rows, rows % base_rows


def test_flat_kernels_split_large_launches():
    """A flat launch keeps its chunk index below 2^31: more chunks take
    several launches over row slices, each indexing its outputs from its
    own first row.  The standalone quantiser (MXFP8 and 1x128 on rows of
    256: 2^26 + 1000 rows, 32 GiB of input) and SiLU-and-mul (1x128 and
    MXFP8 at I = 128: 2^27 + 1000 rows, 64 GiB of input), each input a
    seeded 4096-row block tiled on the GPU; rows on both sides of the split
    against the oracle on the block's rows, bit for bit (MXFP8 SiLU, whose
    fp32 activation the contract holds to a budget: against the same rows
    run as a small launch, bit for bit)."""
    base_rows = 4096
    # standalone quantiser: C = 32 chunks a row, 2^26 rows a launch
    M = (1 << 26) + 1000
    base = inputs.norm_inputs(base_rows, 256, seed=19, x_std=2.0, r_std=None, w_kind="uniform", w_param=0.5)["x"]
    print(f"case flat split: fp8_quant on {M} rows of 256", flush=True)
    x = dev16(base).repeat(M // base_rows + 1, 1)[:M]
    rows, brow = _split_rows(M, 1 << 26, base_rows, 5)
    idx = torch.from_numpy(rows).cuda()
    for mode in (afq.MXFP8, afq.BLOCK128):
        qa = afq.fp8_quant(x, mode)
        torch.cuda.synchronize()
        got_v = qa.values.view(torch.uint8)[idx].cpu().numpy()
        got_s = qa.scales[idx].cpu().numpy()
        del qa
        q, sc = orc.quant(base[brow], orc.BF16, mode)
        assert np.array_equal(got_v, q), mode
        assert np.array_equal(np.ascontiguousarray(got_s).view(np.uint8), np.ascontiguousarray(sc).view(np.uint8)), mode
    del x
    torch.cuda.empty_cache()
    # SiLU-and-mul: C = 16 chunks a row (I = 128), 2^27 rows a launch
    M = (1 << 27) + 1000
    base = inputs.gate_up_inputs(base_rows, 128, seed=20, std=2.0)
    print(f"case flat split: silu_mul_quant on {M} rows of I=128", flush=True)
    gu = dev16(base).repeat(M // base_rows + 1, 1)[:M]
    rows, brow = _split_rows(M, 1 << 27, base_rows, 6)
    idx = torch.from_numpy(rows).cuda()
    for mode in (afq.BLOCK128, afq.MXFP8):
        qa = afq.silu_mul_quant(gu, mode)
        torch.cuda.synchronize()
        got_v = qa.values.view(torch.uint8)[idx].cpu().numpy()
        got_s = qa.scales[idx].cpu().numpy()
        del qa
        if mode == afq.BLOCK128:   # bit-exact against the oracle
            ref = orc.silu_quant(base[brow], mode, want_act=False)
            assert np.array_equal(got_v, ref["values"])
            assert np.array_equal(got_s.view(np.uint32), ref["scales"].view(np.uint32))
        else:                      # the same rows as a small launch, bit for bit
            small = afq.silu_mul_quant(dev16(base[brow]), mode)
            torch.cuda.synchronize()
            assert np.array_equal(got_v, host8(small.values))
            assert np.array_equal(got_s, small.scales.cpu().numpy())
    del gu
    torch.cuda.empty_cache()


# ------------------------------------------------ full-size, every row
@pytest.mark.parametrize("name,M,H,mode,normed", [
    ("headline add + Gemma RMSNorm + MXFP8 + copy", 16384, 6144, "mx", True),
    ("add + Gemma RMSNorm + MXFP8 + copy", 4096, 6144, "mx", True),
    ("add + standard RMSNorm + 1x128", 4096, 4096, "b128", False),
])
def test_full_size_norm_all_rows(name, M, H, mode, normed):
    """The benchmark's norm workloads at full size, launched exactly as
    timed (same inputs, same outputs requested, hence the same row shape):
    every row against the oracle.  Headline and its M = 4096 form: x, r ~
    N(0,3^2), w ~ N(0,0.1^2), seed 1; the 1x128 form: x, r ~ N(0,1),
    w ~ U(0.5,1.5), seed 0, no copy."""
    print(f"case full size {name} M={M} H={H}", flush=True)
    if mode == "mx":
        d = inputs.norm_inputs(M, H, seed=1, x_std=3.0, r_std=3.0, w_kind="normal", w_param=0.1)
        kind = "gemma"
    else:
        d = inputs.norm_inputs(M, H, seed=0, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5)
        kind = "standard"
    gpu = run_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode, want_normed=normed)
    ref = ref_norm(d["x"], d["w"], r=d["r"], kind=kind, mode=mode)
    _report(f"full size {name} M={M}", check_norm(gpu, ref, mode, "bf16", f"full-{mode}-{M}"))
