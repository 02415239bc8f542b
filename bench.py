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
  cpu_baseline the CPU oracle on a bounded sample of the headline workload.

    python bench.py [--steps K] [--warmup W] [--gpus 1] [--no-sweep] [--no-cpu]
    python bench.py --profile    (only the headline kernel and a 1 GiB copy,
                                  for rocprofv3 counter runs)
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
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


# ----------------------------------------------------------- byte formulas
def norm_bytes(M, H, *, residual=True, normed=True, mode="mx", elt=2):
    """Algorithmic HBM bytes of one norm launch: read x (and r), write h,
    the optional copy, the codes and the scales; the weight once."""
    per_row = elt * H                       # x
    if residual:
        per_row += 2 * elt * H              # r in, h out
    if normed:
        per_row += elt * H                  # normed copy
    per_row += H                            # e4m3 codes
    per_row += {"mx": H // 32, "b128": 4 * (H // 128), "pt": 4}[mode]
    return M * per_row + elt * H


def silu_bytes(M, I, *, mode="mx"):
    return M * (4 * I + I + (I // 32 if mode == "mx" else 4 * (I // 128)))


def two_seg_bytes(M, widths=(1536, 512)):
    return sum(norm_bytes(M, n, residual=False, normed=False, mode="pt") for n in widths)


# ------------------------------------------------------------------- helpers
def _dev16(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def _src_hash():
    h = hashlib.sha256()
    for f in ("afq_norm.hip", "afq_device.hpp", "afq_launch.hpp"):
        with open(os.path.join(ROOT, "activation_fp8_quant_amd", "csrc", f), "rb") as fh:
            h.update(fh.read())
    return h.hexdigest()[:16]


def time_events(fn, steps, warmup):
    """Average ms per call of fn over `steps` calls, HIP events on the
    current stream, device synchronised on both sides."""
    import torch
    for _ in range(warmup):
        fn()
    torch.cuda.synchronize()
    s, e = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    s.record()
    for _ in range(steps):
        fn()
    e.record()
    torch.cuda.synchronize()
    return s.elapsed_time(e) / steps


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
                 normed=True, sets=1):
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
                                                residual=ri, want_normed=normed)
            self.sets.append(dict(x=xi, r=ri, out=(proto.values, proto.scales, proto.normed),
                                  rout=proto.residual))
        self.w = w
        self.i = 0
        self.bytes = norm_bytes(M, H, residual=r is not None, normed=normed, mode=mode)
        torch.cuda.synchronize()

    def __call__(self):
        s = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fused_add_rmsnorm_quant(s["x"], self.w, 1e-6, mode=self.mode, kind=self.kind,
                                         residual=s["r"], residual_out=s["rout"], out=s["out"])


class SiluCase:
    def __init__(self, M, I, *, seed, std, mode, sets=1):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        self.mode = {"mx": afq.MXFP8, "b128": afq.BLOCK128}[mode]
        gu = _dev16(inputs.gate_up_inputs(M, I, seed=seed, std=std))
        self.sets = []
        for i in range(sets):
            gi = gu if i == 0 else gu.clone()
            proto = afq.silu_mul_quant(gi, self.mode)
            self.sets.append((gi, (proto.values, proto.scales, None)))
        self.i = 0
        self.bytes = silu_bytes(M, I, mode=mode)
        torch.cuda.synchronize()

    def __call__(self):
        g, out = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.silu_mul_quant(g, self.mode, out=out)


class TwoSegCase:
    def __init__(self, M, *, seed, sets=1):
        import torch
        import activation_fp8_quant_amd as afq
        from activation_fp8_quant_amd import inputs
        self.afq = afq
        segs = inputs.two_segment_inputs(M, (1536, 512), seed=seed)
        buf = np.zeros((M, 2112), np.uint16)
        buf[:, :1536] = segs[0]["x"]
        buf[:, 1536:2048] = segs[1]["x"]
        b = _dev16(buf)
        self.w = [_dev16(s["w"]) for s in segs]
        self.sets = []
        for i in range(sets):
            bi = b if i == 0 else b.clone()
            xs = [bi[:, :1536], bi[:, 1536:2048]]
            outs = afq.fused_add_rmsnorm_quant(xs, self.w, 1e-6, mode=afq.PER_TOKEN,
                                               kind=afq.STANDARD)
            self.sets.append((xs, [(o.values, o.scales, None) for o in outs]))
        self.i = 0
        self.bytes = two_seg_bytes(M)
        torch.cuda.synchronize()

    def __call__(self):
        xs, outs = self.sets[self.i]
        self.i = (self.i + 1) % len(self.sets)
        self.afq.fused_add_rmsnorm_quant(xs, self.w, 1e-6, mode=self.afq.PER_TOKEN,
                                         kind=self.afq.STANDARD, out=outs)


def rotation_sets(ws_bytes, target=1 << 30):
    return max(1, -(-target // max(ws_bytes, 1)))


# ----------------------------------------------------------------- CPU leg
def cpu_baseline(rows=16384):
    """The oracle, as it stands, on a bounded sample of the headline
    workload: `rows` rows of the M = 16384, H = 6144 batch, one oracle call
    per thread over a row range."""
    import oracle as orc
    from activation_fp8_quant_amd import inputs
    H = 6144
    d = inputs.norm_inputs(rows, H, seed=1, x_std=3.0, r_std=3.0, w_kind="normal", w_param=0.1)
    threads = min(os.cpu_count() or 1, 16)
    orc.norm_quant(d["x"][:8], d["w"], residual=d["r"][:8], kind=orc.GEMMA, dtype=orc.BF16,
                   mode=orc.MXFP8, eps=1e-6, threads=1)  # tables, page-in
    t0 = time.perf_counter()
    orc.norm_quant(d["x"], d["w"], residual=d["r"], kind=orc.GEMMA, dtype=orc.BF16,
                   mode=orc.MXFP8, eps=1e-6, threads=threads)
    dt = time.perf_counter() - t0
    b = norm_bytes(rows, H)
    return {"value": round(b / dt / 1e9, 4), "unit": "GB/s", "cores": threads, "kind": "oracle",
            "sample": f"{rows} of the 16384 rows (H=6144), {dt:.2f} s wall on {threads} threads",
            "us_per_row": round(dt * 1e6 / rows, 2)}


# ------------------------------------------------------------------- main
def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=1000)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--profile", action="store_true",
                    help="only the headline kernel and a 1 GiB device copy (counter runs)")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the fused kernels are row-independent and this build "
              "has no multi-GPU path (see DESIGN.md on sharding); run with --gpus 1",
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
        for _ in range(args.warmup + args.steps):
            head()
        src = torch.empty(1 << 29, dtype=torch.int16, device="cuda")  # 1 GiB
        dst = torch.empty_like(src)
        for _ in range(5):
            dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"profile": True, "steps": args.steps, "copy_bytes": 1 << 30}), flush=True)
        return

    torch.cuda.synchronize()
    ms = time_events(head, args.steps, args.warmup)
    gbs = head.bytes / (ms * 1e-3) / 1e9
    print(f"[bench] headline {ms * 1e3:.2f} us/launch, {gbs:.1f} GB/s", file=sys.stderr, flush=True)

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
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": "fused add + Gemma RMSNorm + MXFP8 (1x32 E8M0, e4m3) + bf16 copy",
                   "M": M, "H": H, "seed": 1, "inputs": "x, r ~ N(0,3^2), w ~ N(0,0.1^2) bf16",
                   "bytes_per_launch": head.bytes},
        "us_per_launch": round(ms * 1e3, 2),
        "pct_hbm_peak": round(100.0 * gbs / HBM_PEAK_GBS, 1),
        "roofline": {"bound": "hbm", "achieved": round(gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(gbs / HBM_PEAK_GBS, 4), "traffic": traffic,
                     "kernel": "norm_quant_kernel<bf16, MXFP8, Gemma, 1 chunk/lane, 1 segment>, 768 lanes per row"},
    }
    del head
    torch.cuda.empty_cache()

    if not args.no_sweep:
        sweep = []
        for m in (8, 16, 32, 64, 128, 192):
            c = NormCase(m, 6144, seed=0, x_std=3.0, r_std=1.0, w_kind="normal", w_param=0.1,
                         kind="gemma", mode="mx", normed=True)
            us = graph_time_us(c)
            s = SiluCase(m, 768, seed=0, std=2.0, mode="mx")
            us_s = graph_time_us(s)
            sweep.append({"workload": "norm gemma mx+copy H=6144", "M": m, "us_per_launch": round(us, 2),
                          "GBps": round(c.bytes / us / 1e3, 1), "page_us": PAGE_NORM_US[m],
                          "method": "graph replay 200x after >= 200 ms warm replays, median of 20"})
            sweep.append({"workload": "silu-mul mx I=768", "M": m, "us_per_launch": round(us_s, 2),
                          "GBps": round(s.bytes / us_s / 1e3, 1), "page_us_swiglu_oai": PAGE_SWIGLU_US[m],
                          "method": "graph replay 200x after >= 200 ms warm replays, median of 20"})
            print(f"[bench] M={m}: norm {us:.2f} us, silu {us_s:.2f} us", file=sys.stderr, flush=True)
            del c, s
        big = [
            ("norm gemma mx+copy H=6144", lambda k: NormCase(4096, 6144, seed=1, x_std=3.0, r_std=3.0,
                                                             w_kind="normal", w_param=0.1, kind="gemma",
                                                             mode="mx", sets=k), norm_bytes(4096, 6144), 4096),
            ("norm standard b128 H=4096", lambda k: NormCase(4096, 4096, seed=0, x_std=1.0, r_std=1.0,
                                                             w_kind="uniform", w_param=0.5, kind="standard",
                                                             mode="b128", normed=False, sets=k),
             norm_bytes(4096, 4096, normed=False, mode="b128"), 4096),
            ("silu-mul b128 I=12288", lambda k: SiluCase(4096, 12288, seed=0, std=1.0, mode="b128", sets=k),
             silu_bytes(4096, 12288, mode="b128"), 4096),
            ("two-seg per-token 1536+512", lambda k: TwoSegCase(8192, seed=0, sets=k), two_seg_bytes(8192), 8192),
            ("silu-mul b128 I=3072", lambda k: SiluCase(16384, 3072, seed=1, std=3.0, mode="b128", sets=k),
             silu_bytes(16384, 3072, mode="b128"), 16384),
        ]
        for name, make, ws, m in big:
            k = rotation_sets(ws)
            c = make(k)
            iters = max(2 * k, 20)
            us_c = graph_time_us(c, iters=iters, reps=10)
            sweep.append({"workload": name, "M": m, "us_per_launch": round(us_c, 2),
                          "GBps": round(c.bytes / us_c / 1e3, 1),
                          "pct_hbm_peak": round(100 * c.bytes / us_c / 1e3 / HBM_PEAK_GBS, 1),
                          "method": f"graph replay of {iters} launches over {k} rotating buffer sets "
                                    "after >= 200 ms warm replays, "
                                    "median of 10"})
            print(f"[bench] {name} M={m}: {us_c:.2f} us", file=sys.stderr, flush=True)
            del c
            torch.cuda.empty_cache()
        result["sweep"] = sweep

    if not args.no_cpu:
        result["cpu_baseline"] = cpu_baseline()
        print(f"[bench] cpu baseline {result['cpu_baseline']}", file=sys.stderr, flush=True)

    print(json.dumps(result), flush=True)


if __name__ == "__main__":
    main()
