"""Helpers for the GPU tests: move the seeded host inputs to the device, run
the library through its binding, bring results back as numpy, and compare
them with the oracle under the rules of tests/_compare.py."""
from __future__ import annotations

import os

import numpy as np
import torch

import activation_fp8_quant_amd as afq
import oracle as orc
from tests._compare import check_dtype16, check_quant, scales_u8_or_f32

TORCH16 = {"bf16": torch.bfloat16, "fp16": torch.float16}
ORC_DT = {"bf16": orc.BF16, "fp16": orc.FP16}
MODE = {"mx": afq.MXFP8, "b128": afq.BLOCK128, "pt": afq.PER_TOKEN}
KIND = {"gemma": afq.GEMMA, "standard": afq.STANDARD}
# host threads for the oracle (at most 16: a process driving one GPU is
# commonly given a share of the machine's cores)
HOST_THREADS = max(1, min(os.cpu_count() or 1, 16))


def dev16(bits: np.ndarray, dtype: str = "bf16") -> torch.Tensor:
    t = torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16).view(np.int16))
    return t.view(TORCH16[dtype]).cuda()


def host16(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def host8(t: torch.Tensor) -> np.ndarray:
    return t.detach().contiguous().view(torch.uint8).cpu().numpy()


def check_norm(gpu: dict, ref: dict, mode: str, dtype: str, name: str, requant=True, qin=0):
    """gpu/ref: dict(h, normed, values, scales) numpy.  h exact, normed <= 1
    ulp, codes/scales within the quant budget (every inexact scale explained
    and listed), and the GPU's codes/scales are exactly the oracle quantiser
    applied to the GPU's own rounded row.  With qin = QIN_FP32 (fp32-direct:
    the kernel forms inv, the normed value, the scale and the quotient in the
    same fp32 operations as the oracle) every output is bit-exact."""
    stats = {}
    exact = qin == afq.QIN_FP32
    if gpu.get("h") is not None:
        check_dtype16(gpu["h"], ref["h"], name + ".h", exact=True)
    if gpu.get("normed") is not None:
        stats["normed_1ulp"] = check_dtype16(gpu["normed"], ref["normed"], name + ".normed", exact=exact)
    if exact:
        bad = np.flatnonzero(np.asarray(gpu["values"]).ravel() != np.asarray(ref["values"]).ravel())
        assert bad.size == 0, f"{name}: {bad.size} codes differ (fp32-direct is exact), first at {bad[:5]}"
        gs = np.ascontiguousarray(gpu["scales"], np.float32).view(np.uint32)
        rs = np.ascontiguousarray(ref["scales"], np.float32).view(np.uint32)
        bad = np.flatnonzero(gs.ravel() != rs.ravel())
        assert bad.size == 0, f"{name}: {bad.size} scales differ (fp32-direct is exact), first at {bad[:5]}"
        stats["exact"] = True
        return stats
    stats["codes_1"], stats["scales_bad"], listed = check_quant(
        gpu["values"], gpu["scales"], ref["values"], ref["scales"], MODE[mode], name,
        u=ref.get("normed"), dtype=dtype)
    if listed:
        stats["inexact_scales"] = listed
    if requant and gpu.get("normed") is not None:
        q, s = orc.quant(gpu["normed"], ORC_DT[dtype], MODE[mode], threads=HOST_THREADS)
        assert np.array_equal(q, gpu["values"]), name + ": codes differ from oracle(quant(gpu normed))"
        if MODE[mode] == afq.MXFP8:
            assert np.array_equal(s, gpu["scales"]), name + ": scales differ from oracle(quant(gpu normed))"
        else:
            assert np.array_equal(s.view(np.uint32), np.ascontiguousarray(gpu["scales"], np.float32).view(np.uint32)), \
                name + ": scales differ from oracle(quant(gpu normed))"
    return stats


def run_norm(x, w, *, r=None, kind="gemma", mode="mx", dtype="bf16", eps=1e-6, want_normed=True,
             qin=0):
    xt, wt = dev16(x, dtype), dev16(w, dtype)
    rt = dev16(r, dtype) if r is not None else None
    qa = afq.fused_add_rmsnorm_quant(xt, wt, eps, mode=MODE[mode], kind=KIND[kind], residual=rt,
                                     want_normed=want_normed, quant_input=qin)
    torch.cuda.synchronize()
    return dict(h=host16(qa.residual) if r is not None else None,
                normed=host16(qa.normed) if want_normed else None,
                values=host8(qa.values), scales=scales_u8_or_f32(qa.scales))


def ref_norm(x, w, *, r=None, kind="gemma", mode="mx", dtype="bf16", eps=1e-6, rows=None, qin=0):
    return orc.norm_quant(x, w, residual=r, kind=KIND[kind], dtype=ORC_DT[dtype], mode=MODE[mode],
                          eps=eps, want_normed=True, threads=HOST_THREADS, rows=rows, qin=qin)
