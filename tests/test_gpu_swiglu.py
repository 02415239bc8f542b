"""GPU parity of the clamped SwiGLU + MXFP8 (swiglu_oai_quant) against the
oracle: the pages' benchmark shapes and parameters (vLLM pull request 65478,
"Microbenchmark script": gate_up = randn * 8, [M, 2 * 768], alpha 1.702,
beta 1.0, limit 7.0), every finite bf16 gate, other parameters, extreme
gates, the bf16-first variant, the unfused chain and graph replay."""
import numpy as np
import pytest
import torch

import activation_fp8_quant_amd as afq
import oracle as orc
from activation_fp8_quant_amd import inputs
from tests._compare import check_codes, check_dtype16, check_scales, scales_u8_or_f32
from tests._gpu import dev16, host16, host8

pytestmark = pytest.mark.gpu

ALPHA, BETA, LIMIT = 1.702, 1.0, 7.0


def _report(name, stats):
    print(f"[{name}] " + " ".join(f"{k}={v}" for k, v in stats.items()), flush=True)


def _run(gu, alpha=ALPHA, beta=BETA, limit=LIMIT, qin=afq.QIN_DEFAULT, want_act=True):
    qa = afq.swiglu_oai_quant(dev16(gu), alpha, beta, limit, want_act=want_act, quant_input=qin)
    torch.cuda.synchronize()
    return dict(values=host8(qa.values), scales=scales_u8_or_f32(qa.scales),
                act=host16(qa.normed) if want_act else None)


def _run_act(act, gu, want_act=True):
    """One of the two MXFP8 activations with the pages' parameters."""
    if act == "swiglu":
        return _run(gu, want_act=want_act)
    qa = afq.silu_mul_quant(dev16(gu), afq.MXFP8, want_act=want_act)
    torch.cuda.synchronize()
    return dict(values=host8(qa.values), scales=scales_u8_or_f32(qa.scales),
                act=host16(qa.normed) if want_act else None)


def _ref_act(act, gu):
    if act == "swiglu":
        return orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, threads=8)
    return orc.silu_quant(gu, orc.MXFP8, threads=8)


def _check(gpu, ref, name):
    n1 = check_codes(gpu["values"], ref["values"], name)
    nb, _ = check_scales(gpu["scales"], ref["scales"], 0, name)
    out = dict(codes_1=n1, scales_bad=nb)
    if gpu["act"] is not None:
        out["act_1ulp"] = check_dtype16(gpu["act"], ref["act"], name + " act")
    return out


@pytest.mark.parametrize("want_act", [False, True])
@pytest.mark.parametrize("M", [8, 16, 64, 192, 300])
def test_swiglu_mx_pages_shapes(M, want_act):
    print(f"case swiglu pages shape M={M} copy={want_act}", flush=True)
    gu = inputs.gate_up_inputs(M, 768, seed=0, std=8.0)
    gpu = _run(gu, want_act=want_act)
    ref = orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, threads=8)
    _report(f"swiglu-mx M={M} copy={want_act}", _check(gpu, ref, "swiglu-mx"))


@pytest.mark.parametrize("I,M", [(3072, 33), (2176, 9), (32, 5), (12288, 3)])
def test_swiglu_mx_widths(I, M):
    print(f"case swiglu width I={I} M={M}", flush=True)
    gu = inputs.gate_up_inputs(M, I, seed=3, std=8.0)
    gpu = _run(gu)
    ref = orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, threads=8)
    _check(gpu, ref, f"swiglu-mx I={I}")


def test_swiglu_mx_all_gates():
    """Every finite bf16 gate times ten up values: inside the clamp (1,
    -2.75, 2^-10, 3e-3, 2^-100), beyond it (96, -2^40, 1e30) and where
    beta cancels up (-1, giving zero activations)."""
    print("case swiglu all gates", flush=True)
    gu = _all_gates_rows([1.0, -2.75, 2.0 ** -10, 3e-3, 2.0 ** -100, 96.0, -(2.0 ** 40), 1e30, -1.0,
                          6.9375])
    gpu = _run(gu)
    ref = orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, threads=8)
    stats = _check(gpu, ref, "swiglu-mx all gates")
    _report("swiglu-mx all gates x 10 ups", dict(elements=int(gu.shape[0] * 128), **stats))


# Quantising MXFP8 launches without the bf16 copy and of at most 131,072
# 8-element chunks take the 4-values-per-lane form of the activation
# kernel; larger ones, and launches that write the copy, the 8-per-lane form.
def _all_gates_rows(ups, tiles=1):
    c = np.arange(1 << 16, dtype=np.uint32)
    gates = c[((c >> 7) & 0xFF) != 0xFF].astype(np.uint16)
    pad = (-gates.size) % 128
    g = np.concatenate([gates, np.zeros(pad, np.uint16)]).reshape(-1, 128)
    ub = inputs.to_bits(np.array(ups))
    return np.concatenate([np.concatenate([g, np.full_like(g, u)], axis=1) for u in ub] * tiles, axis=0)


@pytest.mark.parametrize("act", ["silu", "swiglu"])
def test_mx_activation_forms_agree_on_all_gates(act):
    """Every finite bf16 gate times eight up values: the 4-per-lane form
    (no copy requested, 81,600 chunks) and the 8-per-lane form (copy
    requested) give bit-identical codes and scales, within the budget of
    the oracle."""
    print(f"case forms agree {act}", flush=True)
    gu = _all_gates_rows([1.0, -2.75, 2.0 ** -10, 3e-3, 96.0, -(2.0 ** 40), 2.0 ** -100, 1e30])
    four = _run_act(act, gu, want_act=False)
    eight = _run_act(act, gu, want_act=True)
    assert np.array_equal(four["values"], eight["values"])
    assert np.array_equal(four["scales"], eight["scales"])
    _report(f"{act}-mx all gates, 4 per lane", _check(four, _ref_act(act, gu), f"{act}-mx 4/lane"))


@pytest.mark.parametrize("act", ["silu", "swiglu"])
@pytest.mark.parametrize("M", [1365, 1366])
def test_mx_activation_at_the_form_boundary(act, M):
    """Rows 1365 and 1366 at I = 768 (131,040 and 131,136 chunks), no copy:
    the two kernel forms on either side of the switch, against the oracle."""
    print(f"case mx activation boundary {act} M={M}", flush=True)
    gu = inputs.gate_up_inputs(M, 768, seed=6, std=8.0 if act == "swiglu" else 2.0)
    _report(f"{act}-mx M={M}", _check(_run_act(act, gu, want_act=False), _ref_act(act, gu),
                                      f"{act}-mx boundary"))


@pytest.mark.parametrize("act", ["silu", "swiglu"])
def test_mx_activation_all_gates_8_per_lane_without_copy(act):
    """Every finite bf16 gate times four up values, tiled five times so that
    a launch without the copy (163,200 chunks) takes the 8-per-lane form."""
    print(f"case all gates 8 per lane {act}", flush=True)
    gu = _all_gates_rows([1.0, -2.75, 96.0, 2.0 ** -10], tiles=5)
    _report(f"{act}-mx all gates 8 per lane",
            _check(_run_act(act, gu, want_act=False), _ref_act(act, gu), f"{act}-mx all gates 8/lane"))


@pytest.mark.parametrize("M", [8, 192])
def test_swiglu_bf16_first_without_copy(M):
    """The bf16-first variant in the 4-per-lane form equals its 8-per-lane
    form (with the copy) bit for bit."""
    gu = inputs.gate_up_inputs(M, 768, seed=8, std=8.0)
    four = _run(gu, qin=afq.QIN_BF16, want_act=False)
    eight = _run(gu, qin=afq.QIN_BF16, want_act=True)
    assert np.array_equal(four["values"], eight["values"])
    assert np.array_equal(four["scales"], eight["scales"])
    qo, so = orc.quant(eight["act"], orc.BF16, orc.MXFP8)
    assert np.array_equal(qo, four["values"]) and np.array_equal(so, four["scales"])


@pytest.mark.parametrize("alpha,beta,limit", [(1.0, 0.0, float("inf")), (1.0, 0.5, 2.5),
                                              (1.702, 1.0, 7.3), (0.25, -3.0, 100.0),
                                              (-0.5, 1.0, 4.0), (3.5, 0.0, 1e-3)])
def test_swiglu_other_parameters(alpha, beta, limit):
    """Other parameters: plain SiLU-and-mul (alpha 1, beta 0, no clamp, also
    checked against the SiLU oracle), a limit that is not a bf16 value (7.3),
    a negative alpha, a tiny limit."""
    print(f"case swiglu params {alpha} {beta} {limit}", flush=True)
    gu = inputs.gate_up_inputs(64, 512, seed=5, std=8.0)
    gpu = _run(gu, alpha, beta, limit)
    ref = orc.swiglu_oai_quant(gu, alpha, beta, limit, threads=8)
    _check(gpu, ref, f"swiglu-mx params {alpha},{beta},{limit}")
    if (alpha, beta, limit) == (1.0, 0.0, float("inf")):
        sref = orc.silu_quant(gu, orc.MXFP8, threads=8)
        for k in ("values", "scales", "act"):
            assert np.array_equal(ref[k], sref[k])


def test_swiglu_extreme_gates():
    """Gates far below -80 / alpha (the fp64 path), huge gates under an
    infinite limit, zeros of both signs."""
    print("case swiglu extreme gates", flush=True)
    rng = np.random.default_rng(11)
    g = rng.standard_normal((6, 256)) * 30.0
    g[0, :64] = -rng.uniform(47, 60, 64)        # alpha gc below -80
    g[1, :] = rng.uniform(-60, -45, 256)         # whole blocks of tiny activations
    g[2, :32] = [1e30, -1e30, 3e38, -3e38, 0.0, -0.0, 1e-38, -1e-38] * 4
    u = rng.standard_normal((6, 256)) * 8.0
    gu = np.concatenate([inputs.to_bits(g), inputs.to_bits(u)], axis=1)
    for limit in (LIMIT, float("inf")):
        gpu = _run(gu, limit=limit)
        ref = orc.swiglu_oai_quant(gu, ALPHA, BETA, limit)
        if limit == LIMIT:
            _check(gpu, ref, "swiglu-mx extreme")
        else:
            # huge gates times up overflow fp32 there: compare the groups
            # whose activation stays finite
            fin = (ref["act"] & 0x7FFF) < 0x7F80
            okg = fin.reshape(6, -1, 32).all(axis=2)
            assert np.array_equal(gpu["scales"][okg], ref["scales"][okg])
            okel = np.repeat(okg, 32, axis=1)
            d = np.abs(gpu["values"][okel].astype(np.int64) - ref["values"][okel].astype(np.int64))
            assert (d > 0).sum() <= 1
            check_dtype16(gpu["act"][fin], ref["act"][fin], "swiglu-mx extreme act")


def test_swiglu_bf16_first_and_unfused_chain():
    """The bf16-first variant quantises the kernel's own bf16 activation
    (codes and scales equal the oracle quantiser applied to it); the unfused
    chain (copy-only launch, then fp8_quant) equals it bit for bit; the
    default fusion differs from the chain in a few % of codes, as [P1]
    reports for its own kernels (1.9-2.4 %)."""
    print("case swiglu bf16-first / chain", flush=True)
    gu = inputs.gate_up_inputs(192, 768, seed=0, std=8.0)
    g = dev16(gu)
    bf = afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True, quant_input=afq.QIN_BF16)
    fused = afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True)
    plain = afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, quantize=False)
    assert plain.values is None and plain.scales is None
    q = afq.fp8_quant(plain.normed, afq.MXFP8)
    torch.cuda.synchronize()
    act = host16(bf.normed)
    qo, so = orc.quant(act, orc.BF16, orc.MXFP8)
    assert np.array_equal(qo, host8(bf.values)) and np.array_equal(so, scales_u8_or_f32(bf.scales))
    assert torch.equal(plain.normed.view(torch.int16), bf.normed.view(torch.int16))
    assert torch.equal(plain.normed.view(torch.int16), fused.normed.view(torch.int16))
    assert torch.equal(q.values.view(torch.uint8), bf.values.view(torch.uint8))
    assert torch.equal(q.scales, bf.scales)
    ref = orc.swiglu_oai_quant(gu, ALPHA, BETA, LIMIT, qin=orc.QIN_BF16, threads=8)
    _check(dict(values=host8(bf.values), scales=scales_u8_or_f32(bf.scales), act=act), ref,
           "swiglu-mx bf16-first")
    differ = (q.values.view(torch.uint8) != fused.values.view(torch.uint8)).float().mean().item()
    sdiffer = (q.scales != fused.scales).float().mean().item()
    _report("swiglu mx: unfused chain vs fp32 fusion", dict(codes_differ=round(differ, 4),
                                                            scales_differ=round(sdiffer, 4)))
    assert differ < 0.1


def test_swiglu_graph_replay_and_determinism():
    """Captured launches equal eager ones on every replay, and repeated
    launches are bitwise identical."""
    print("case swiglu graph replay", flush=True)
    gu = inputs.gate_up_inputs(64, 768, seed=4, std=8.0)
    g = dev16(gu)
    eager = afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True)
    torch.cuda.synchronize()
    out = (torch.empty_like(eager.values), torch.empty_like(eager.scales),
           torch.empty_like(eager.normed))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True, out=out)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True, out=out)
    for _ in range(3):
        for t in out:
            t.view(torch.uint8).fill_(0x5A)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        assert torch.equal(out[0].view(torch.uint8), eager.values.view(torch.uint8))
        assert torch.equal(out[1], eager.scales)
        assert torch.equal(out[2].view(torch.int16), eager.normed.view(torch.int16))
    for _ in range(5):
        again = afq.swiglu_oai_quant(g, ALPHA, BETA, LIMIT, want_act=True)
        torch.cuda.synchronize()
        assert torch.equal(again.values.view(torch.uint8), eager.values.view(torch.uint8))
        assert torch.equal(again.scales, eager.scales)
