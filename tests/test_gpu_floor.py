"""The two-segment per-token norm (RMSNorm + per-token FP8 of rows of 1536
+ 512, 8192 rows) against the floor of its own memory traffic: a probe
kernel (tests/probe) makes the same loads and stores, one wavefront a row,
with the arithmetic replaced by a wavefront-wide sum that every store still
waits for.  Both are timed as bench.py times the launch: graph replay over
rotated buffer sets of at least 1 GiB."""
import numpy as np
import pytest
import torch

import bench
from tests.test_gpu_instructions import _probe

pytestmark = pytest.mark.gpu


def test_two_segment_per_token_against_its_memory_pattern():
    """The fused launch takes little more than the probe that moves its
    bytes without computing (printed with -s); it must stay within a quarter
    of it."""
    M, pitch = 8192, 2112 * 2
    k = bench.rotation_sets(bench.two_seg_bytes(M))
    case = bench.TwoSegCase(M, seed=0, sets=k)
    fused_us = bench.graph_time_us(case, iters=max(200, k), reps=10)
    del case
    L = _probe()
    sets = []
    for _ in range(k):
        sets.append((torch.empty((M, 2112), dtype=torch.bfloat16, device="cuda").normal_(),
                     torch.empty((M, 1536), dtype=torch.uint8, device="cuda"),
                     torch.empty((M, 512), dtype=torch.uint8, device="cuda"),
                     torch.empty(M, dtype=torch.float32, device="cuda"),
                     torch.empty(M, dtype=torch.float32, device="cuda")))
    turn = [0]

    def probe():
        x, q0, q1, s0, s1 = sets[turn[0]]
        turn[0] = (turn[0] + 1) % k
        rc = L.afqp_rows_pattern(x.data_ptr(), pitch, q0.data_ptr(), q1.data_ptr(), s0.data_ptr(),
                                 s1.data_ptr(), M, 192, 256, torch.cuda.current_stream().cuda_stream)
        assert rc == 0

    probe_us = bench.graph_time_us(probe, iters=max(200, k), reps=10)
    gbs = bench.two_seg_bytes(M) / 1e3
    print(f"\ntwo-segment per-token, {M} rows, {k} buffer sets: fused {fused_us:.2f} us "
          f"({gbs / fused_us:.0f} GB/s), its memory pattern alone {probe_us:.2f} us "
          f"({gbs / probe_us:.0f} GB/s)", flush=True)
    assert np.isfinite(fused_us) and np.isfinite(probe_us)
    assert fused_us < 1.25 * probe_us
