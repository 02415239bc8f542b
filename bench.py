#!/usr/bin/env python3
"""Benchmark of the fused activation FP8 quantisation kernels on one MI355X.

Headline (the JSON `value`): fused add + Gemma RMSNorm + MXFP8 + bf16 copy,
H = 6144, M = 16384 rows (the bandwidth-bound prefill shape), as achieved
algorithmic HBM GB/s.  A step is one launch of that kernel over the batch;
inputs are resident in HBM before timing starts.  Timing: W untimed
launches (default 1000, about 150 ms: after an idle phase the GPU's clocks
take some tens of ms of sustained work to settle), then K launches
bracketed by HIP events on the launch stream (and a device synchronisation
on both sides).

Also reported, in the same JSON line:
  sweep        us/launch at decode sizes M = 8..192 by the graph-replay
               method (200 launches captured in a HIP graph, at least 200 ms
               of untimed replays, then the median of 20 timed replays / 200)
               for the fused norm and the SiLU-and-mul + MXFP8 kernel, next
               to the figures the pages print for their own kernels
               (context only); and the other
               workloads (1x128 norm / SiLU, per-token two-segment norm)
               timed with buffer rotation so that no launch reads data
               another launch left in the 256 MB last-level cache.
  roofline     the dominant kernel against the 8 TB/s HBM peak.
  device_copy  a 1 GiB device-to-device copy: the achievable streaming rate,
               and the headline as a fraction of it.
  cpu_baseline the CPU oracle on a bounded sample of the headline workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-cpu]
    python bench.py --profile [NAME]   (one workload -- the headline, or one of
                                        PROFILE_WORKLOADS -- and a 1 GiB copy,
                                        for rocprofv3 trace and counter runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import statistics
import sys
import threading
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "HBM GB/s (% peak) + µs/launch, fused add+RMSNorm+MXFP8, H=6144, M=8..16384"
HBM_PEAK_GBS = 8000.0

# pages' per-launch figures (MI355X, their Triton kernels; context, not targets)
PAGE_NORM_US = {8: 2.71, 16: 2.77, 32: 2.80, 64: 2.96, 128: 3.29, 192: 3.65}
PAGE_SWIGLU_US = {8: 1.83, 16: 1.93, 32: 1.95, 64: 1.94, 128: 1.90, 192: 1.95}
# the same table's unfused columns: norm + separate quant (2 launches) and
# the time the fusion saves; swiglu + separate quant and its saving
PAGE_NORM_CHAIN_US = {8: 4.27, 16: 4.32, 32: 4.40, 64: 4.79, 128: 5.55, 192: 6.94}
PAGE_NORM_SAVED_US = {8: 1.56, 16: 1.55, 32: 1.60, 64: 1.83, 128: 2.26, 192: 3.29}
PAGE_SWIGLU_CHAIN_US = {8: 3.82, 16: 3.96, 32: 3.97, 64: 4.00, 128: 4.06, 192: 4.04}
PAGE_SWIGLU_SAVED_US = {8: 1.99, 16: 2.03, 32: 2.02, 64: 2.06, 128: 2.16, 192: 2.09}


# ----------------------------------------------------------- byte formulas
def norm_bytes(M, H, *, residual=True, normed=True, mode="mx", elt=2, quant=True):
    """Algorithmic HBM bytes of one norm launch: read x (and r), write h,
    the optional copy, the codes and the scales (not for a copy-only
    launch); the weight once."""
    per_row = elt * H                       # x
    if residual:
        per_row += 2 * elt * H              # r in, h out
    if normed:
        per_row += elt * H                  # normed copy
    if quant:
        per_row += H                        # e4m3 codes
        per_row += {"mx": H // 32, "b128": 4 * (H // 128), "pt": 4}[mode]
    return M * per_row + elt * H


def silu_bytes(M, I, *, mode="mx", quant=True):
    """Read [M, 2I] bf16; write codes and scales, or (copy-only) the bf16
    activation."""
    if not quant:
        return M * (4 * I + 2 * I)
    return M * (4 * I + I + (I // 32 if mode == "mx" else 4 * (I // 128)))


def two_seg_bytes(M, widths=(1536, 512), quant=True):
    return sum(norm_bytes(M, n, residual=False, normed=not quant, mode="pt", quant=quant)
               for n in widths)


# ------------------------------------------------------------------- helpers
def _dev16(bits, dtype="bf16"):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).cuda()


def _code_only(text: str) -> str:
    """C++ source without its comments and with runs of white space made one
    space: what the compiler sees, so that a comment edit does not count as
    a change of the kernel."""
    text = re.sub(r"/\*.*?\*/", " ", text, flags=re.S)
    text = re.sub(r"//[^\n]*", " ", text)
    return " ".join(text.split())


def _src_hash():
    """Hash of the norm kernel's sources (comments and layout excluded), to
    tell whether stored counter figures still describe the kernel."""
    h = hashlib.sha256()
    for f in ("afq_norm.hip", "afq_device.hpp", "afq_launch.hpp", "afq_shape.hpp"):
        with open(os.path.join(ROOT, "activation_fp8_quant_amd", "csrc", f), encoding="utf-8") as fh:
            h.update(_code_only(fh.read()).encode())
    return h.hexdigest()[:16]


def time_events(fn, steps, warmup, warm_s=0.2):
    """Average ms per call of fn over `steps` calls, HIP events on the
    current stream, device synchronised on both sides.  Untimed warm-up
    first: at least `warmup` calls and at least `warm_s` seconds of them
    (after an idle phase the GPU's clocks take some tens of ms of sustained
    work to settle).  Returns (ms per call, warm-up calls made)."""
    import torch
    t0 = time.perf_counter()
    n = 0
    while n < warmup or time.perf_counter() - t0 < warm_s:
        fn()
        n += 1
        if n % 64 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps, n


def graph_time_us(fn, iters=200, reps=20, warm_s=0.2):
    """us per launch by graph replay: capture `iters` launches, replay for
    at least `warm_s` seconds untimed (the GPU's clocks take some tens of ms
    of sustained work to settle after an idle phase such as building the
    inputs), then the median of `reps` timed replays divided by `iters`."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(iters):
                fn()
    torch.cuda.current_stream().wait_stream(st)
    t0 = time.perf_counter()
    n = 0
    while n < 3 or time.perf_counter() - t0 < warm_s:
        g.replay()
        n += 1
        if n % 8 == 0:
            torch.cuda.synchronize()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        g.replay()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) * 1000.0 / iters)
    return statistics.median(ts)


# --------------------------------------------------------------- workloads
class NormCase:
    """Preallocated buffers of one fused-norm workload (k rotation sets)."""

    def __init__(self, M, H, *, seed, x_std, r_std, w_kind, w_param, kind, mode,
                 normed=True, sets=1, qin=0, quantize=True):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq, self.M, self.H, self.mode_name = afq, M, H, mode
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128, "pt": afq.PER_TOKEN}[mode]
        self.kind = {"gemma": afq.GEMMA, "standard": afq.STANDARD}[kind]
        d = inputs.norm_inputs(M, H, seed=seed, x_std=x_std, r_std=r_std, w_kind=w_kind,
                               w_param=w_param)
        x, w = _dev16(d["x"]), _dev16(d["w"])
        r = _dev16(d["r"]) if d["r"] is not None else None
        self.sets = []
        for i in range(sets):
            xi = x if i == 0 else x.clone()
            ri = None if r is None else (r if i == 0 else r.clone())
            proto = afq.fused_add_rmsnorm_quant(xi, w, 1e-6, mode=self.mode, kind=self.kind,
                                                residual=ri, want_normed=normed, quant_input=qin,
                                                quantize=quantize)
            self.sets.append(dict(x=xi, r=ri, out=(proto.values, proto.scales, proto.normed),
                                  rout=proto.residual))
        self.w = w
        self.qin = qin
        self.quantize = quantize
        self.i = 0
        self.bytes = norm_bytes(M, H, residual=r is not None, normed=normed or not quantize,
                                mode=mode, quant=quantize)
        torch.cuda.synchronize()

    def __call__(self):
        s = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fused_add_rmsnorm_quant(s["x"], self.w, 1e-6, mode=self.mode, kind=self.kind,
                                         residual=s["r"], residual_out=s["rout"], out=s["out"],
                                         quant_input=self.qin, quantize=self.quantize)

    def prepared(self):
        """The same launch on buffer set 0, marshalled once (afq.prepare)."""
        s = self.sets[0]
        return self.afq.prepare(self.afq.fused_add_rmsnorm_quant, s["x"], self.w, 1e-6, mode=self.mode,
                                kind=self.kind, residual=s["r"], residual_out=s["rout"], out=s["out"],
                                quant_input=self.qin, quantize=self.quantize)


class SiluCase:
    """SiLU-and-mul + quant, or with swiglu = (alpha, beta, limit) the
    clamped SwiGLU + MXFP8."""

    def __init__(self, M, I, *, seed, std, mode, sets=1, qin=0, swiglu=None, quantize=True):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128}[mode]
        self.swiglu = swiglu
        self.qin = qin
        self.quantize = quantize
        gu = _dev16(inputs.gate_up_inputs(M, I, seed=seed, std=std))
        self.sets = []
        for i in range(sets):
            gi = gu if i == 0 else gu.clone()
            proto = self._launch(gi, None)
            self.sets.append((gi, (proto.values, proto.scales, proto.normed if not quantize else None)))
        self.i = 0
        self.bytes = silu_bytes(M, I, mode=mode, quant=quantize)
        torch.cuda.synchronize()

    def _launch(self, g, out):
        if self.swiglu:
            return self.afq.swiglu_oai_quant(g, *self.swiglu, out=out, quant_input=self.qin,
                                             quantize=self.quantize)
        return self.afq.silu_mul_quant(g, self.mode, out=out, quant_input=self.qin,
                                       quantize=self.quantize)

    def __call__(self):
        g, out = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self._launch(g, out)

    def prepared(self):
        """The same launch on buffer set 0, marshalled once (afq.prepare)."""
        g, out = self.sets[0]
        if self.swiglu:
            return self.afq.prepare(self.afq.swiglu_oai_quant, g, *self.swiglu, out=out,
                                    quant_input=self.qin, quantize=self.quantize)
        return self.afq.prepare(self.afq.silu_mul_quant, g, self.mode, out=out, quant_input=self.qin,
                                quantize=self.quantize)


class TwoSegCase:
    def __init__(self, M, *, seed, sets=1, dtype="bf16", quantize=True):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        segs = inputs.two_segment_inputs(M, (1536, 512), seed=seed, dtype=dtype)
        buf = np.zeros((M, 2112), np.uint16)
        buf[:, :1536] = segs[0]["x"]
        buf[:, 1536:2048] = segs[1]["x"]
        b = _dev16(buf, dtype)
        self.w = [_dev16(s["w"], dtype) for s in segs]
        self.sets = []
        for i in range(sets):
            bi = b if i == 0 else b.clone()
            xs = [bi[:, :1536], bi[:, 1536:2048]]
            outs = afq.fused_add_rmsnorm_quant(xs, self.w, 1e-6, mode=afq.PER_TOKEN,
                                               kind=afq.STANDARD, quantize=quantize)
            self.sets.append((xs, [(o.values, o.scales, o.normed) for o in outs]))
        self.quantize = quantize
        self.i = 0
        self.bytes = two_seg_bytes(M, quant=quantize)
        torch.cuda.synchronize()

    def __call__(self):
        xs, outs = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fused_add_rmsnorm_quant(xs, self.w, 1e-6, mode=self.afq.PER_TOKEN,
                                         kind=self.afq.STANDARD, out=outs, quantize=self.quantize)


class NormChainCase:
    """The unfused chain on this library's kernels: a copy-only add + RMSNorm
    launch (residual and normed rows), then the standalone quantiser on its
    rows -- two launches per call."""

    def __init__(self, M, H, *, seed, x_std, r_std, w_kind, w_param, kind, mode, sets=1):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128, "pt": afq.PER_TOKEN}[mode]
        self.kind = {"gemma": afq.GEMMA, "standard": afq.STANDARD}[kind]
        d = inputs.norm_inputs(M, H, seed=seed, x_std=x_std, r_std=r_std, w_kind=w_kind,
                               w_param=w_param)
        x, self.w, r = _dev16(d["x"]), _dev16(d["w"]), _dev16(d["r"])
        self.sets = []
        for i in range(sets):
            xi, ri = (x, r) if i == 0 else (x.clone(), r.clone())
            plain = afq.fused_add_rmsnorm_quant(xi, self.w, 1e-6, mode=self.mode, kind=self.kind,
                                                residual=ri, quantize=False)
            q = afq.fp8_quant(plain.normed, self.mode)
            self.sets.append(dict(x=xi, r=ri, rout=plain.residual, normed=plain.normed,
                                  out=(q.values, q.scales, None)))
        self.i = 0
        self.bytes = M * (8 * H + 2 * H + H + H // 32) + 2 * H
        torch.cuda.synchronize()

    def __call__(self):
        s = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fused_add_rmsnorm_quant(s["x"], self.w, 1e-6, mode=self.mode, kind=self.kind,
                                         residual=s["r"], residual_out=s["rout"], quantize=False,
                                         out=(None, None, s["normed"]))
        self.afq.fp8_quant(s["normed"], self.mode, out=s["out"])


class SiluChainCase:
    """The unfused SiLU chain on this library's kernels: a copy-only
    SiLU-and-mul launch (bf16 activation), then the standalone quantiser.
    With swiglu = (alpha, beta, limit): the clamped SwiGLU's chain."""

    def __init__(self, M, I, *, seed, std, mode, sets=1, swiglu=None):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128}[mode]
        self.swiglu = swiglu
        gu = _dev16(inputs.gate_up_inputs(M, I, seed=seed, std=std))
        self.sets = []
        for i in range(sets):
            gi = gu if i == 0 else gu.clone()
            plain = self._act(gi, None)
            q = afq.fp8_quant(plain.normed, self.mode)
            self.sets.append((gi, plain.normed, (q.values, q.scales, None)))
        self.i = 0
        self.bytes = M * (4 * I + 2 * I + 2 * I + I + I // 32)
        torch.cuda.synchronize()

    def _act(self, g, act):
        out = None if act is None else (None, None, act)
        if self.swiglu:
            return self.afq.swiglu_oai_quant(g, *self.swiglu, quantize=False, out=out)
        return self.afq.silu_mul_quant(g, self.mode, quantize=False, out=out)

    def __call__(self):
        g, act, out = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self._act(g, act)
        self.afq.fp8_quant(act, self.mode, out=out)


class QuantCase:
    """The standalone quantiser on a bf16 [M, H] activation (the separate
    quant kernel of an unfused chain)."""

    def __init__(self, M, H, *, seed, std, mode, sets=1):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128, "pt": afq.PER_TOKEN}[mode]
        x = _dev16(inputs.to_bits(np.random.default_rng(seed).standard_normal((M, H)) * std))
        self.sets = []
        for i in range(sets):
            xi = x if i == 0 else x.clone()
            proto = afq.fp8_quant(xi, self.mode)
            self.sets.append((xi, (proto.values, proto.scales, None)))
        self.i = 0
        self.bytes = M * (2 * H + H + {"mx": H // 32, "b128": 4 * (H // 128), "pt": 4}[mode])
        torch.cuda.synchronize()

    def __call__(self):
        x, out = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fp8_quant(x, self.mode, out=out)


def rotation_sets(ws_bytes, target=1 << 30):
    return max(1, -(-target // max(ws_bytes, 1)))


def eager_single_us(fn, reps=50):
    """us of one launch timed alone: events around it on an idle GPU,
    median over `reps` (includes the launch latency and the host's time to
    issue it: the binding's checks and marshalling, or for a prepared launch
    only the C call)."""
    import torch
    fn()
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        s.record()
        fn()
        e.record()
        torch.cuda.synchronize()
        ts.append(s.elapsed_time(e) * 1000.0)
    return statistics.median(ts)


# ------------------------------------------------------------- the sweep
DECODE_M = (8, 16, 32, 64, 128, 192)


def run_sweep():
    """Every configuration and row count of the measurement plan, as a list
    of records.  Hot: 200 launches over one buffer set (the pages' method;
    the decode rows compare with their figures).  Rotated: one replay cycle
    walks k buffer sets with k * (working set) >= 1 GiB, so that no launch
    reads what an earlier one left in the 256 MB last-level cache; used for
    every working set of at least 1 MiB (smaller launches are bound by
    launch latency, and would need tens of thousands of buffer sets)."""
    import torch

    def log(msg):
        print(f"[bench] {msg}", file=sys.stderr, flush=True)

    out = []

    def rec(cfg, name, make, M, ws, *, hot=False, **extra):
        k = 1 if hot or ws < (1 << 20) else rotation_sets(ws)
        case = make(k)
        us = graph_time_us(case, iters=max(200, k), reps=20 if k == 1 else 10)
        r = {"config": cfg, "workload": name, "M": M, "us_per_launch": round(us, 2),
             "GBps": round(case.bytes / us / 1e3, 1),
             "cache": "hot (one buffer set)" if k == 1 else f"rotated over {k} buffer sets"}
        if M >= 4096:
            r["pct_hbm_peak"] = round(100 * case.bytes / us / 1e3 / HBM_PEAK_GBS, 1)
        if "eager" in extra:
            extra["eager_single_us"] = round(eager_single_us(case), 2)
            extra["eager_single_prepared_us"] = round(eager_single_us(case.prepared()), 2)
            del extra["eager"]
        r.update(extra)
        out.append(r)
        log(f"{cfg} {name} M={M} {r['cache']}: {us:.2f} us")
        del case
        torch.cuda.empty_cache()
        return r

    def copy_floor(r, make_copy, ws):
        """Time the copy-only launch of the same workload (same kernel, same
        row shape rules, the rounded copy written instead of codes and
        scales) with buffer rotation, and attach it to the fused record: the
        in-repo figure for what the memory pattern alone achieves."""
        k = rotation_sets(ws)
        case = make_copy(k)
        us = graph_time_us(case, iters=max(200, k), reps=10)
        gbs = case.bytes / us / 1e3
        r["copy_only"] = {"us_per_launch": round(us, 2), "bytes": case.bytes, "GBps": round(gbs, 1),
                          "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 1),
                          "fused_GBps_over_copy_only": round(r["GBps"] / gbs, 3)}
        log(f"  copy-only: {us:.2f} us, {gbs:.0f} GB/s")
        del case
        torch.cuda.empty_cache()

    # trivial-kernel floor: a one-element fill, timed the same way
    t = torch.zeros(1, device="cuda")
    floor = graph_time_us(lambda: t.fill_(1.0))
    out.append({"config": "floor", "workload": "one-element torch fill (trivial kernel)",
                "us_per_launch": round(floor, 2), "cache": "hot (one buffer set)"})
    log(f"trivial-kernel floor {floor:.2f} us")

    c1 = "add + Gemma RMSNorm + MXFP8 + bf16 copy, H=6144"

    def norm_c1(M):
        return lambda k: NormCase(M, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal",
                                  w_param=0.1, kind="gemma", mode="mx", normed=True, sets=k)

    for M in DECODE_M:
        ws = norm_bytes(M, 6144)
        fused = rec("C1", c1, norm_c1(M), M, ws, hot=True, page_us=PAGE_NORM_US[M], eager=True)
        if ws >= (1 << 20):
            rec("C1", c1, norm_c1(M), M, ws)
        fused_s = rec("C2", "SiLU-and-mul + MXFP8, I=768",
                      lambda k, M=M: SiluCase(M, 768, seed=0, std=2.0, mode="mx", sets=k), M,
                      silu_bytes(M, 768), hot=True, page_us_swiglu_oai=PAGE_SWIGLU_US[M], eager=True)
        rec("f1", "standalone MXFP8 quant of a bf16 [M, 6144] (the separate quant)",
            lambda k, M=M: QuantCase(M, 6144, seed=0, std=3.0, mode="mx", sets=k), M,
            M * (3 * 6144 + 6144 // 32), hot=True)
        # the unfused chains on this library's kernels, and what the fusion saves
        ch = rec("f1", "unfused chain: copy-only add + Gemma RMSNorm, then MXFP8 quant "
                 "(2 launches), H=6144",
                 lambda k, M=M: NormChainCase(M, 6144, seed=0, x_std=3.0, r_std=1.0,
                                              w_kind="normal", w_param=0.1, kind="gemma",
                                              mode="mx", sets=k),
                 M, M * (11 * 6144 + 6144 // 32), hot=True, page_us=PAGE_NORM_CHAIN_US[M])
        ch["saved_us"] = round(ch["us_per_launch"] - fused["us_per_launch"], 2)
        ch["page_saved_us"] = PAGE_NORM_SAVED_US[M]
        ch = rec("f1", "unfused chain: copy-only SiLU-and-mul, then MXFP8 quant (2 launches), "
                 "I=768", lambda k, M=M: SiluChainCase(M, 768, seed=0, std=2.0, mode="mx", sets=k),
                 M, M * (9 * 768 + 768 // 32), hot=True, page_us_swiglu_oai=PAGE_SWIGLU_CHAIN_US[M])
        ch["saved_us"] = round(ch["us_per_launch"] - fused_s["us_per_launch"], 2)
        ch["page_saved_us_swiglu_oai"] = PAGE_SWIGLU_SAVED_US[M]
    # the clamped SwiGLU the pages time (swiglu_oai(gu, 1.702, 1.0, 7.0) on
    # gu = randn * 8): fused, the unfused chain, what the fusion saves, and
    # how many codes and scales the fp32 fusion changes against the chain
    import activation_fp8_quant_amd as afq
    oai = (1.702, 1.0, 7.0)
    for M in DECODE_M:
        fz = rec("f2", "clamped SwiGLU (swiglu_oai 1.702, 1.0, 7.0) + MXFP8, I=768, gate_up ~ N(0, 8^2)",
                 lambda k, M=M: SiluCase(M, 768, seed=0, std=8.0, mode="mx", sets=k, swiglu=oai), M,
                 silu_bytes(M, 768), hot=True, page_us=PAGE_SWIGLU_US[M], eager=True)
        ch = rec("f2", "unfused chain: copy-only clamped SwiGLU, then MXFP8 quant (2 launches), I=768",
                 lambda k, M=M: SiluChainCase(M, 768, seed=0, std=8.0, mode="mx", sets=k, swiglu=oai),
                 M, M * (9 * 768 + 768 // 32), hot=True, page_us=PAGE_SWIGLU_CHAIN_US[M])
        ch["saved_us"] = round(ch["us_per_launch"] - fz["us_per_launch"], 2)
        ch["page_saved_us"] = PAGE_SWIGLU_SAVED_US[M]
        from activation_fp8_quant_amd import inputs
        g = _dev16(inputs.gate_up_inputs(M, 768, seed=0, std=8.0))
        f = afq.swiglu_oai_quant(g, *oai)
        q = afq.fp8_quant(afq.swiglu_oai_quant(g, *oai, quantize=False).normed, afq.MXFP8)
        fz["codes_differ_vs_chain"] = round((f.values.view(torch.uint8) != q.values.view(torch.uint8))
                                            .float().mean().item(), 4)
        fz["scales_differ_vs_chain"] = round((f.scales != q.scales).float().mean().item(), 4)
    for M in (256, 1024, 2048):
        rec("C1", c1, norm_c1(M), M, norm_bytes(M, 6144))
    def c3a(M, quantize=True):
        return lambda k: NormCase(M, 4096, seed=0, x_std=1.0, r_std=1.0, w_kind="uniform",
                                  w_param=0.5, kind="standard", mode="b128", normed=False, sets=k,
                                  quantize=quantize)

    for M in (1, 32, 256, 4096):
        r = rec("C3a", "add + standard RMSNorm + 1x128, H=4096", c3a(M), M,
                norm_bytes(M, 4096, normed=False, mode="b128"))
        if M == 4096:
            copy_floor(r, c3a(M, quantize=False), norm_bytes(M, 4096, mode="b128", quant=False))

    def c3b(M, quantize=True):
        return lambda k: SiluCase(M, 12288, seed=0, std=1.0, mode="b128", sets=k, quantize=quantize)

    for M in (1, 32, 256, 4096):
        r = rec("C3b", "SiLU-and-mul + 1x128, I=12288", c3b(M), M, silu_bytes(M, 12288, mode="b128"))
        if M == 4096:
            copy_floor(r, c3b(M, quantize=False), silu_bytes(M, 12288, quant=False))
    for dt in ("bf16", "fp16"):
        for M in (1, 8, 64, 1024, 8192):
            r = rec("C4", f"RMSNorm + per-token, two segments 1536 + 512, {dt}",
                    lambda k, M=M, dt=dt: TwoSegCase(M, seed=0, sets=k, dtype=dt), M, two_seg_bytes(M))
            if M == 8192:
                copy_floor(r, lambda k, M=M, dt=dt: TwoSegCase(M, seed=0, sets=k, dtype=dt,
                                                                quantize=False),
                           two_seg_bytes(M, quant=False))

    def c5a(quantize=True):
        return lambda k: NormCase(4096, 6144, seed=1, x_std=3.0, r_std=3.0, w_kind="normal",
                                  w_param=0.1, kind="gemma", mode="mx", sets=k, quantize=quantize)

    r = rec("C5a", c1 + " (M = 16384 is the headline)", c5a(), 4096, norm_bytes(4096, 6144))
    copy_floor(r, c5a(quantize=False), norm_bytes(4096, 6144, quant=False))
    # rounding-point variants: fp32-direct 1x128 norm, bf16-first MXFP8 SiLU
    for M in (32, 4096):
        rec("f2", "add + standard RMSNorm + 1x128, fp32-direct (quantise the fp32 normed value), H=4096",
            lambda k, M=M: NormCase(M, 4096, seed=0, x_std=1.0, r_std=1.0, w_kind="uniform",
                                    w_param=0.5, kind="standard", mode="b128", normed=False, sets=k,
                                    qin=afq.QIN_FP32),
            M, norm_bytes(M, 4096, normed=False, mode="b128"))
    for M in (8, 192):
        rec("f2", "SiLU-and-mul + MXFP8, bf16-first (quantise the bf16 activation), I=768",
            lambda k, M=M: SiluCase(M, 768, seed=0, std=2.0, mode="mx", sets=k, qin=afq.QIN_BF16), M,
            silu_bytes(M, 768), hot=True)
    def c5b(quantize=True):
        return lambda k: SiluCase(16384, 3072, seed=1, std=3.0, mode="b128", sets=k,
                                  quantize=quantize)

    r = rec("C5b", "SiLU-and-mul + 1x128, I=3072", c5b(), 16384, silu_bytes(16384, 3072, mode="b128"))
    copy_floor(r, c5b(quantize=False), silu_bytes(16384, 3072, quant=False))
    # the standalone per-token quantiser (the separate quant of a per-token chain)
    for M in (8, 1024, 4096):
        rec("f1", "standalone per-token quant of a bf16 [M, 8192]",
            lambda k, M=M: QuantCase(M, 8192, seed=0, std=3.0, mode="pt", sets=k), M,
            M * (3 * 8192 + 4), hot=M <= 64)
    return out


# Workloads of `--profile NAME` (besides the headline): the rotated bench
# workloads, built exactly as the sweep builds them.
def _prof_norm_b128(qin=0):
    import activation_fp8_quant_amd as afq
    ws = norm_bytes(4096, 4096, normed=False, mode="b128")
    return NormCase(4096, 4096, seed=0, x_std=1.0, r_std=1.0, w_kind="uniform", w_param=0.5,
                    kind="standard", mode="b128", normed=False, sets=rotation_sets(ws),
                    qin=afq.QIN_FP32 if qin else 0)


PROFILE_WORKLOADS = {
    "norm_mx_m4096": lambda: NormCase(4096, 6144, seed=1, x_std=3.0, r_std=3.0, w_kind="normal",
                                      w_param=0.1, kind="gemma", mode="mx",
                                      sets=rotation_sets(norm_bytes(4096, 6144))),
    "norm_b128_h4096": lambda: _prof_norm_b128(),
    "norm_b128_f32q_h4096": lambda: _prof_norm_b128(qin=1),
    "twoseg_pt_m8192": lambda: TwoSegCase(8192, seed=0, sets=rotation_sets(two_seg_bytes(8192))),
    "norm_mx_m1024": lambda: NormCase(1024, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal",
                                      w_param=0.1, kind="gemma", mode="mx",
                                      sets=rotation_sets(norm_bytes(1024, 6144))),
    "silu_b128_i12288": lambda: SiluCase(4096, 12288, seed=0, std=1.0, mode="b128",
                                         sets=rotation_sets(silu_bytes(4096, 12288, mode="b128"))),
    "silu_b128_i3072": lambda: SiluCase(16384, 3072, seed=1, std=3.0, mode="b128",
                                        sets=rotation_sets(silu_bytes(16384, 3072, mode="b128"))),
    "quant_pt_h8192_m1024": lambda: QuantCase(1024, 8192, seed=0, std=3.0, mode="pt",
                                              sets=rotation_sets(1024 * 3 * 8192)),
    # decode sizes, hot (one buffer set), launched by graph replay as the
    # sweep times them
    "norm_mx_m8": lambda: NormCase(8, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal",
                                   w_param=0.1, kind="gemma", mode="mx"),
    "silu_mx_i768_m8": lambda: SiluCase(8, 768, seed=0, std=2.0, mode="mx"),
    "swiglu_mx_i768_m8": lambda: SiluCase(8, 768, seed=0, std=8.0, mode="mx",
                                          swiglu=(1.702, 1.0, 7.0)),
    "quant_mx_h6144_m8": lambda: QuantCase(8, 6144, seed=0, std=3.0, mode="mx"),
}
PROFILE_BY_GRAPH = {"norm_mx_m8", "silu_mx_i768_m8", "swiglu_mx_i768_m8", "quant_mx_h6144_m8"}


def replay_launches(fn, launches, per_graph=200):
    """Run about `launches` launches of fn as replays of a captured graph of
    `per_graph` launches (the decode timing method), for profiler runs."""
    import torch
    fn()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    st = torch.cuda.Stream()
    st.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(st):
        with torch.cuda.graph(g, stream=st):
            for _ in range(per_graph):
                fn()
    torch.cuda.current_stream().wait_stream(st)
    for i in range(max(1, -(-launches // per_graph))):
        g.replay()
        if i % 8 == 7:
            torch.cuda.synchronize()
    torch.cuda.synchronize()


# ------------------------------------------------------- host cost per call
def host_overhead(calls=2000, reps=5):
    """Host time of one eager call at a decode size: perf_counter over
    `calls` back-to-back calls with preallocated outputs and no
    synchronisation in between (each launch runs on the GPU in less time
    than the host takes to issue it, so the host is what is timed), median
    of `reps` runs.  For the decode norm (add + Gemma RMSNorm + MXFP8 + copy,
    8 x 6144) and SiLU-and-mul + MXFP8 (8 x 768): the binding's entry point
    with out= given; the same launch prepared once (afq.prepare: only the C
    ABI call and the kernel launch remain); and a one-element torch fill."""
    import torch
    import activation_fp8_quant_amd as afq
    from activation_fp8_quant_amd import inputs

    def per_call(fn):
        for _ in range(200):
            fn()
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            t0 = time.perf_counter()
            for _ in range(calls):
                fn()
            ts.append((time.perf_counter() - t0) / calls * 1e6)
            torch.cuda.synchronize()
        return round(statistics.median(ts), 2)

    d = inputs.norm_inputs(8, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1)
    x, w, r = _dev16(d["x"]), _dev16(d["w"]), _dev16(d["r"])
    kw = dict(mode=afq.MXFP8, kind=afq.GEMMA, residual=r)
    p = afq.fused_add_rmsnorm_quant(x, w, 1e-6, want_normed=True, **kw)
    out, rout = (p.values, p.scales, p.normed), p.residual
    norm_full = per_call(lambda: afq.fused_add_rmsnorm_quant(x, w, 1e-6, residual_out=rout, out=out, **kw))
    norm_prep = per_call(afq.prepare(afq.fused_add_rmsnorm_quant, x, w, 1e-6, residual_out=rout,
                                     out=out, **kw))
    gu = _dev16(inputs.gate_up_inputs(8, 768, seed=0, std=2.0))
    q = afq.silu_mul_quant(gu, afq.MXFP8)
    sout = (q.values, q.scales, None)
    silu_full = per_call(lambda: afq.silu_mul_quant(gu, afq.MXFP8, out=sout))
    silu_prep = per_call(afq.prepare(afq.silu_mul_quant, gu, afq.MXFP8, out=sout))
    t = torch.zeros(1, device="cuda")
    fill = per_call(lambda: t.fill_(1.0))
    return {"method": f"perf_counter over {calls} eager calls, no sync in between, median of {reps}",
            "norm_mx_8x6144": {"entry_point_us": norm_full, "prepared_us": norm_prep},
            "silu_mx_8x768": {"entry_point_us": silu_full, "prepared_us": silu_prep},
            "torch_fill_one_element_us": fill}


# ----------------------------------------------------------------- CPU leg
def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


# The oracle's row threads are capped at 16: a process that drives one GPU
# is commonly given a share of a larger machine's cores, and the cap keeps
# the baseline comparable between machines.  The record states the cap,
# the machine's CPU count and the CPUs this process may use.
CPU_THREAD_CAP = 16


def cpu_baseline(rows=16384, reps=5):
    """The oracle, as it stands, on a bounded sample of the headline
    workload: `rows` rows of the M = 16384, H = 6144 batch, split over row
    ranges on T threads (T = the CPUs this process may run on, capped at
    CPU_THREAD_CAP).  One warm-up call, then the median of `reps` timed calls
    (steady clock); also one thread on the first 1024 rows (median of 3)."""
    import oracle as orc
    from activation_fp8_quant_amd import inputs
    H = 6144
    d = inputs.norm_inputs(rows, H, seed=1, x_std=3.0, r_std=3.0, w_kind="normal", w_param=0.1)
    try:
        usable = len(os.sched_getaffinity(0))
    except AttributeError:  # pragma: no cover
        usable = os.cpu_count() or 1
    threads = max(1, min(usable, CPU_THREAD_CAP))

    def call(r, t):
        t0 = time.perf_counter()
        orc.norm_quant(d["x"][:r], d["w"], residual=d["r"][:r], kind=orc.GEMMA, dtype=orc.BF16,
                       mode=orc.MXFP8, eps=1e-6, threads=t)
        return time.perf_counter() - t0

    call(rows, threads)                                   # warm-up (tables, page-in)
    ts = [call(rows, threads) for _ in range(reps)]
    dt = statistics.median(ts)
    b = norm_bytes(rows, H)
    r1 = min(rows, 1024)
    dt1 = statistics.median([call(r1, 1) for _ in range(3)])
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of the 16384 rows (H=6144): 1 warm-up call, median of {reps} calls "
                      f"({dt:.2f} s each) on {threads} threads",
            "us_per_row": round(dt * 1e6 / rows, 2),
            "times_s": [round(t, 3) for t in ts],
            "host_cpus": os.cpu_count(), "usable_cpus": usable, "thread_cap": CPU_THREAD_CAP,
            "cpu_model": _cpu_model(),
            "one_thread": {"GBps": round(norm_bytes(r1, H) / dt1 / 1e9, 4),
                           "us_per_row": round(dt1 * 1e6 / r1, 1), "rows": r1}}


# ------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", nargs="?", const="headline", default=None,
                    choices=["headline"] + sorted(PROFILE_WORKLOADS),
                    help="only one workload (default: the headline) and a 1 GiB device copy "
                         "(for rocprofv3 trace and counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: rows are independent and the library has no "
              "multi-GPU path (a row-sharded launch per GPU needs no exchange); run with --gpus 1",
              file=sys.stderr, flush=True)
        sys.exit(2)

    import torch
    import activation_fp8_quant_amd as afq
    afq.load()
    torch.cuda.init()

    M, H = 16384, 6144
    head = NormCase(M, H, seed=1, x_std=3.0, r_std=3.0, w_kind="normal", w_param=0.1,
                    kind="gemma", mode="mx", normed=True)
    print(f"[bench] headline inputs ready ({head.bytes / 1e6:.1f} MB per launch)", file=sys.stderr, flush=True)

    if args.profile:
        work = head
        if args.profile != "headline":
            del head
            torch.cuda.empty_cache()
            work = PROFILE_WORKLOADS[args.profile]()
        if args.profile in PROFILE_BY_GRAPH:
            replay_launches(work, args.warmup + args.steps)
        else:
            for _ in range(args.warmup + args.steps):
                work()
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": args.profile, "steps": args.steps, "warmup": args.warmup,
                          "bytes_per_launch": work.bytes, "copy_bytes": 1 << 30}), flush=True)
        return

    torch.cuda.synchronize()
    ms, warm_calls = time_events(head, args.steps, args.warmup)
    head_bytes = head.bytes
    gbs = head_bytes / (ms * 1e-3) / 1e9
    print(f"[bench] headline {ms * 1e3:.2f} us/launch, {gbs:.1f} GB/s", file=sys.stderr, flush=True)

    # device-copy ceiling: torch's 1 GiB device-to-device copy (reads and
    # writes 1 GiB), timed like the headline right after it
    src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")
    dst = torch.empty_like(src)
    copy_ms, _ = time_events(lambda: dst.copy_(src), 50, 100)
    copy_gbs = 2 * (1 << 30) / (copy_ms * 1e-3) / 1e9
    del src, dst
    print(f"[bench] 1 GiB device copy {copy_ms * 1e3:.1f} us, {copy_gbs:.1f} GB/s", file=sys.stderr, flush=True)

    # the headline's copy-only launch (the same kernel without codes and
    # scales: read x, r; write h and the copy), timed the same way: what the
    # memory pattern alone achieves
    del head
    torch.cuda.empty_cache()
    plain = NormCase(M, H, seed=1, x_std=3.0, r_std=3.0, w_kind="normal", w_param=0.1,
                     kind="gemma", mode="mx", normed=True, quantize=False)
    pms, _ = time_events(plain, args.steps, args.warmup)
    pgbs = plain.bytes / (pms * 1e-3) / 1e9
    head_copy_only = {"us_per_launch": round(pms * 1e3, 2), "bytes": plain.bytes, "GBps": round(pgbs, 1),
                      "pct_hbm_peak": round(100.0 * pgbs / HBM_PEAK_GBS, 1),
                      "fused_GBps_over_copy_only": round(gbs / pgbs, 3)}
    del plain
    torch.cuda.empty_cache()
    print(f"[bench] headline copy-only {pms * 1e3:.2f} us/launch, {pgbs:.1f} GB/s", file=sys.stderr, flush=True)

    traffic = None
    tpath = os.path.join(ROOT, "profiles", "traffic_norm_mx_h6144_m16384.json")
    if os.path.exists(tpath):
        with open(tpath) as f:
            t = json.load(f)
        if t.get("src_hash") == _src_hash():
            traffic = t.get("traffic_bytes_per_launch")

    result = {
        "metric": METRIC, "value": round(gbs, 1), "unit": "GB/s", "n_gpus": 1,
        "steps": args.steps, "warmup": args.warmup, "ms_per_step": round(ms, 5),
        "warmup_calls_made": warm_calls,
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused add + Gemma RMSNorm + MXFP8 (1x32 E8M0, e4m3) + bf16 copy",
                   "M": M, "H": H, "seed": 1, "inputs": "x, r ~ N(0,3^2), w ~ N(0,0.1^2) bf16",
                   "bytes_per_launch": head_bytes},
        "us_per_launch": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "copy_only": head_copy_only,
        "device_copy": {"GBps": round(copy_gbs, 1), "pct_hbm_peak": round(100.0 * copy_gbs / HBM_PEAK_GBS, 1),
                        "headline_pct_of_copy": round(100.0 * gbs / copy_gbs, 1),
                        "method": "torch 1 GiB device-to-device copy, 100 warm-up + 50 timed, HIP events"},
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "norm_quant_kernel<bf16, MXFP8, Gemma, 1 chunk/lane, 1 segment>, 768 lanes per row"},
    }
    if not args.no_sweep:
        result["host_overhead"] = host_overhead()
        print(f"[bench] host cost per call {result['host_overhead']}", file=sys.stderr, flush=True)
        sweep = run_sweep()
        result["sweep"] = sweep

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
        print(f"[bench] cpu baseline {result['cpu_baseline']}", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
