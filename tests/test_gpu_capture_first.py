"""The first norm launch of a process may be inside a HIP-graph capture.

The launcher reads the device's compute-unit count once per device (the
row-shape rule counts whole rows per CU); that first read then happens
during capture.  A fresh child process (the cache is per process) captures
its very first norm launch in a graph, replays it and compares with an
eager launch.
"""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))

CHILD = r"""
import torch
import activation_fp8_quant_amd as afq
x = torch.randn(1024, 6144, device="cuda", dtype=torch.bfloat16)
w = torch.randn(6144, device="cuda", dtype=torch.bfloat16)
out = (torch.empty(1024, 6144, dtype=torch.float8_e4m3fn, device="cuda"),
       torch.empty(1024, 192, dtype=torch.uint8, device="cuda"),
       torch.empty(1024, 6144, dtype=torch.bfloat16, device="cuda"))
s = torch.cuda.Stream()
g = torch.cuda.CUDAGraph()
with torch.cuda.graph(g, stream=s):
    afq.fused_add_rmsnorm_quant(x, w, 1e-6, want_normed=True, out=out)
for _ in range(3):
    g.replay()
torch.cuda.synchronize()
ref = afq.fused_add_rmsnorm_quant(x, w, 1e-6, want_normed=True)
torch.cuda.synchronize()
assert torch.equal(ref.values.view(torch.uint8), out[0].view(torch.uint8))
assert torch.equal(ref.scales, out[1])
assert torch.equal(ref.normed.view(torch.int16), out[2].view(torch.int16))
print("capture-first ok", flush=True)
"""


@pytest.mark.gpu
def test_first_norm_launch_inside_graph_capture():
    print("[capture-first] child process", flush=True)
    r = subprocess.run([sys.executable, "-c", CHILD], capture_output=True, text=True,
                       timeout=300, cwd=ROOT, env=dict(os.environ, PYTHONPATH=ROOT))
    print(r.stdout, flush=True)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "capture-first ok" in r.stdout
