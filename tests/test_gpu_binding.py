"""The Python binding on the GPU: a launch prepared once (afq.prepare)
equals the entry point's own launch, follows in-place changes of its input
buffers from call to call, and launches on the stream it is given."""
import numpy as np
import pytest
import torch

import activation_fp8_quant_amd as afq
from activation_fp8_quant_amd import inputs
from tests._gpu import dev16

pytestmark = pytest.mark.gpu


def _bytes(t):
    return None if t is None else t.view(torch.uint8).clone()


def _same(a, b):
    for f in ("values", "scales", "normed", "residual"):
        x, y = getattr(a, f), getattr(b, f)
        assert (x is None) == (y is None), f
        if x is not None:
            assert torch.equal(_bytes(x), _bytes(y)), f


def test_prepared_norm_follows_its_inputs():
    d = inputs.norm_inputs(16, 6144, seed=51, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    x, w, r = dev16(d["x"]), dev16(d["w"]), dev16(d["r"])
    kw = dict(mode=afq.MXFP8, kind=afq.GEMMA, residual=r, want_normed=True)
    call = afq.prepare(afq.fused_add_rmsnorm_quant, x, w, 1e-6, **kw)
    assert isinstance(call, afq.PreparedLaunch)
    for step in range(3):
        got = call()
        ref = afq.fused_add_rmsnorm_quant(x, w, 1e-6, **kw)
        torch.cuda.synchronize()
        _same(got, ref)
        x.mul_(-0.5).add_(0.25)              # new contents, same buffer
    s = torch.cuda.Stream()
    with torch.cuda.stream(s):
        x.mul_(2.0)
        got = call(stream=s)
        ref = afq.fused_add_rmsnorm_quant(x, w, 1e-6, **kw)
    s.synchronize()
    _same(got, ref)


@pytest.mark.parametrize("entry", ["silu", "swiglu", "quant", "two_segment"])
def test_prepared_launches_equal_entry_points(entry):
    if entry in ("silu", "swiglu"):
        gu = dev16(inputs.gate_up_inputs(24, 768, seed=52, std=2.0))
        fn, args, kw = ((afq.silu_mul_quant, (gu, afq.MXFP8), dict(want_act=True)) if entry == "silu"
                        else (afq.swiglu_oai_quant, (gu, 1.702, 1.0, 7.0), dict(want_act=True)))
        src = gu
    elif entry == "quant":
        src = torch.from_numpy(np.random.default_rng(53).standard_normal((24, 4096)).astype(np.float32)).cuda()
        fn, args, kw = afq.fp8_quant, (src, afq.PER_TOKEN), {}
    else:
        segs = inputs.two_segment_inputs(300, (1536, 512), seed=54)
        xs, ws = [dev16(sg["x"]) for sg in segs], [dev16(sg["w"]) for sg in segs]
        fn, args, kw = afq.fused_add_rmsnorm_quant, (xs, ws, 1e-6), dict(mode=afq.PER_TOKEN, kind=afq.STANDARD)
        src = xs[0]
    call = afq.prepare(fn, *args, **kw)
    for step in range(2):
        got = call()
        ref = fn(*args, **kw)
        torch.cuda.synchronize()
        if isinstance(got, list):
            for g, r_ in zip(got, ref):
                _same(g, r_)
        else:
            _same(got, ref)
        src.mul_(0.75)


def test_prepare_rejects_bad_use():
    x = torch.zeros((4, 256), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(256, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        afq.prepare(torch.add, x, x)
    with pytest.raises(ValueError):
        afq.prepare(afq.fused_add_rmsnorm_quant, x, w, 1e-6, stream=torch.cuda.current_stream())
    with pytest.raises(ValueError):   # checked at prepare time, before any launch
        afq.prepare(afq.fused_add_rmsnorm_quant, x, w.cpu(), 1e-6)


def test_prepared_launches_in_a_graph():
    """Prepared launches (norm with residual and copy, SiLU-and-mul)
    captured into a HIP graph on the capture stream, then replayed three
    times with new input contents written in place between replays (and the
    outputs poisoned): every replay equals the entry points' eager launches
    on the same inputs.  The residual is not updated in place here, so each
    replay starts from the same residual."""
    d = inputs.norm_inputs(24, 4096, seed=52, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    x, w, r = dev16(d["x"]), dev16(d["w"]), dev16(d["r"])
    gu = dev16(inputs.gate_up_inputs(24, 768, seed=52, std=2.0))
    kw = dict(mode=afq.MXFP8, kind=afq.GEMMA, residual=r, want_normed=True)
    norm = afq.prepare(afq.fused_add_rmsnorm_quant, x, w, 1e-6, **kw)
    silu = afq.prepare(afq.silu_mul_quant, gu, afq.BLOCK128)
    torch.cuda.synchronize()
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    g = torch.cuda.CUDAGraph()
    with torch.cuda.stream(s):
        with torch.cuda.graph(g, stream=s):
            got_n = norm(stream=s)
            got_s = silu(stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    for rep in range(3):
        x.mul_(-0.75).add_(0.5)
        gu.mul_(1.25)
        for t in (got_n.values, got_n.scales, got_n.normed, got_n.residual, got_s.values, got_s.scales):
            t.view(torch.uint8).fill_(0xA5)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        _same(got_n, afq.fused_add_rmsnorm_quant(x, w, 1e-6, **kw))
        _same(got_s, afq.silu_mul_quant(gu, afq.BLOCK128))
        torch.cuda.synchronize()
