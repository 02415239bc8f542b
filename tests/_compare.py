"""Comparison rules between the GPU path and the oracle.

Agreement required (the contract of the library):
  * bf16 / fp16 outputs: at most 1 unit in the last place apart (distance in
    the monotone integer order of the encoding), bit-exact where stated;
  * scales: exact in at least 99.9 % of groups (at least all but one in small
    tests); the rest off by one E8M0 step, one fp32 ulp, or -- for fp32
    scales -- explained by a one-ulp difference of the rounded activation
    (checked separately by re-quantising the GPU's own rounded row);
  * e4m3 codes: equal, or one code apart in at most 0.1 % of elements
    (at most one element in small tests).  0x00 and 0x80 are both zero.
"""
from __future__ import annotations

import math

import numpy as np


def ord16(bits: np.ndarray) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.int64)
    mag = b & 0x7FFF
    return np.where(b & 0x8000, -mag, mag)


def ord8(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    mag = c & 0x7F
    return np.where(c & 0x80, -mag, mag)


def ord32(f: np.ndarray) -> np.ndarray:
    b = np.ascontiguousarray(f, dtype=np.float32).view(np.uint32).astype(np.int64)
    mag = b & 0x7FFFFFFF
    return np.where(b & 0x80000000, -mag, mag)


def budget(n: int, frac: float = 1e-3) -> int:
    return max(1, math.floor(frac * n))


def check_dtype16(gpu, ref, name, max_ulp=1, exact=False):
    d = np.abs(ord16(gpu) - ord16(ref))
    if exact:
        bad = np.flatnonzero(d)
        assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[:5]}"
    else:
        assert d.max(initial=0) <= max_ulp, f"{name}: max ulp distance {d.max()}"
    return int((d != 0).sum())


def check_codes(gpu, ref, name):
    d = np.abs(ord8(gpu) - ord8(ref))
    n1 = int((d == 1).sum())
    assert d.max(initial=0) <= 1, f"{name}: code distance {d.max()} at {np.argwhere(d > 1)[:5].tolist()}"
    assert n1 <= budget(d.size), f"{name}: {n1} of {d.size} codes one step apart"
    return n1


def check_scales(gpu, ref, mode, name):
    """mode 0: uint8 E8M0 bytes; else fp32."""
    if mode == 0:
        d = np.abs(np.asarray(gpu, np.int64) - np.asarray(ref, np.int64))
        assert d.max(initial=0) <= 1, f"{name}: E8M0 off by {d.max()}"
    else:
        gb = np.ascontiguousarray(gpu, np.float32).view(np.uint32)
        rb = np.ascontiguousarray(ref, np.float32).view(np.uint32)
        d = (gb != rb).astype(np.int64)
    nbad = int((d != 0).sum())
    assert nbad <= budget(d.size), f"{name}: {nbad} of {d.size} scales inexact"
    return nbad


def scales_u8_or_f32(t):
    """torch scales tensor -> numpy (uint8 or float32)."""
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.uint8:
        return a.numpy()
    return a.float().numpy()
