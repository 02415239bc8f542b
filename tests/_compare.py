"""Comparison rules between the GPU path and the oracle.

Agreement required (the contract of the library):
  * bf16 / fp16 outputs: at most 1 unit in the last place apart (distance in
    the monotone integer order of the encoding), bit-exact where stated;
  * scales: exact in at least 99.9 % of groups, that is at most
    floor(n / 1000) inexact among the n groups a check covers, unless the
    test states its own budget.  Every inexact scale is listed and must be
    explained:
      - E8M0 bytes: one exponent step apart;
      - fp32 scales: one fp32 ulp apart, or the reading R14 case: the group's
        largest activation rounded to the neighbouring dtype value on the GPU,
        so the scale is fl32(A'/448) with A' the next or previous dtype value
        of the oracle's group amax A (the oracle's rounded activation is
        passed in to decide this; without it only the one-ulp case counts);
  * e4m3 codes: equal, or one code apart in at most 0.1 % of elements
    (floor(n / 1000), unless the test states its budget).  0x00 and 0x80 are
    both zero.
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
    """Inexact groups (or one-apart codes) the contract admits among n."""
    return math.floor(frac * n)


def decode16(bits: np.ndarray, dtype: str) -> np.ndarray:
    """uint16 bit patterns of bf16 / fp16 -> float32 values (exact)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    if dtype == "bf16":
        return (b.astype(np.uint32) << 16).view(np.float32)
    return b.view(np.float16).astype(np.float32)


def check_dtype16(gpu, ref, name, max_ulp=1, exact=False):
    d = np.abs(ord16(gpu) - ord16(ref))
    if exact:
        bad = np.flatnonzero(d)
        assert bad.size == 0, f"{name}: {bad.size} elements differ, first at {bad[:5]}"
    else:
        assert d.max(initial=0) <= max_ulp, f"{name}: max ulp distance {d.max()}"
    return int((d != 0).sum())


def check_codes(gpu, ref, name, allowed=None):
    """Codes equal, or one apart in at most `allowed` elements (default
    floor(n / 1000)).  Returns the number one apart."""
    d = np.abs(ord8(gpu) - ord8(ref))
    n1 = int((d == 1).sum())
    assert d.max(initial=0) <= 1, f"{name}: code distance {d.max()} at {np.argwhere(d > 1)[:5].tolist()}"
    lim = budget(d.size) if allowed is None else allowed
    assert n1 <= lim, f"{name}: {n1} of {d.size} codes one step apart (budget {lim})"
    return n1


def _r14_scales(u_bits: np.ndarray, dtype: str, ngroups: int):
    """For each group of the oracle's rounded activation u [M, cols]: the
    fp32 scales fl32(A'/448) of the amax A moved one dtype value down and up
    (numpy float32 division is the IEEE one).  Returns two [M, ngroups]
    float32 arrays (NaN where the neighbour does not exist)."""
    u = np.ascontiguousarray(u_bits, dtype=np.uint16)
    M, cols = u.shape
    mag = (u & 0x7FFF).reshape(M, ngroups, cols // ngroups)
    a = mag.max(axis=2).astype(np.int64)                        # |A| bit pattern (orders like |A|)
    top = 0x7F7F if dtype == "bf16" else 0x7BFF                 # largest finite magnitude
    lo = np.where(a > 0, a - 1, 0).astype(np.uint16)
    hi = np.minimum(a + 1, top).astype(np.uint16)
    s_lo = decode16(lo, dtype) / np.float32(448.0)
    s_hi = decode16(hi, dtype) / np.float32(448.0)
    s_lo[a == 0] = np.nan
    s_hi[a >= top] = np.nan
    return s_lo.astype(np.float32), s_hi.astype(np.float32)


def check_scales(gpu, ref, mode, name, *, u=None, dtype=None, allowed=None):
    """mode 0: uint8 E8M0 bytes; else fp32 scales [M, groups].

    Every inexact scale is explained (see the module docstring) and listed
    in the returned report; at most `allowed` (default floor(n / 1000)) may
    be inexact.  `u` / `dtype`: the oracle's rounded activation [M, cols]
    (bit patterns) and its dtype, to recognise the R14 case.
    Returns (number inexact, list of (flat index, explanation))."""
    listed = []
    if mode == 0:
        d = np.abs(np.asarray(gpu, np.int64) - np.asarray(ref, np.int64))
        assert d.max(initial=0) <= 1, f"{name}: E8M0 off by {d.max()} at {np.argwhere(d > 1)[:5].tolist()}"
        for i in np.flatnonzero(d):
            listed.append((int(i), "one E8M0 step"))   # explained further by check_quant
        n = d.size
    else:
        g = np.ascontiguousarray(gpu, np.float32)
        r = np.ascontiguousarray(ref, np.float32)
        n = r.size
        bad = np.flatnonzero(g.view(np.uint32).ravel() != r.view(np.uint32).ravel())
        if bad.size:
            dist = np.abs(ord32(g).ravel() - ord32(r).ravel())
            s_lo = s_hi = None
            if u is not None:
                groups = r.reshape(r.shape[0], -1).shape[1]
                s_lo, s_hi = _r14_scales(u, dtype, groups)
                s_lo, s_hi = s_lo.ravel().view(np.uint32), s_hi.ravel().view(np.uint32)
            gb = g.view(np.uint32).ravel()
            for i in bad:
                if dist[i] == 1:
                    listed.append((int(i), "one fp32 ulp"))
                elif s_lo is not None and gb[i] in (s_lo[i], s_hi[i]):
                    listed.append((int(i), "R14: amax one dtype value away"))
                else:
                    raise AssertionError(
                        f"{name}: scale {i} is {float(g.ravel()[i])!r}, oracle {float(r.ravel()[i])!r} "
                        f"({dist[i]} fp32 ulps apart, not explained by a one-ulp amax flip)")
    lim = budget(n) if allowed is None else allowed
    assert len(listed) <= lim, f"{name}: {len(listed)} of {n} scales inexact (budget {lim}): {listed[:10]}"
    return len(listed), listed


def _moved_group_quant(u_row: np.ndarray, lo: int, hi: int, up: bool, dtype: str, mode: int):
    """The oracle's quantisation of one group of the oracle's rounded row
    with its largest-magnitude elements moved one dtype value up (or down):
    returns (codes of the group, scale)."""
    import oracle as orc
    g = np.array(u_row[lo:hi], dtype=np.uint16)
    mag = g & 0x7FFF
    a = int(mag.max())
    top = 0x7F7F if dtype == "bf16" else 0x7BFF
    b = a + 1 if up else a - 1
    if b < 0 or b > top:
        return None, None
    sel = mag == a
    g[sel] = (g[sel] & 0x8000) | np.uint16(b)
    q, sc = orc.quant(g[None, :], orc.BF16 if dtype == "bf16" else orc.FP16, mode)
    return q[0], sc[0]


def check_quant(gpu_values, gpu_scales, ref_values, ref_scales, mode, name, *, u=None, dtype=None,
                allowed_scales=None, allowed_codes=None):
    """Codes and scales of one quantised tensor [M, cols] against the
    oracle's.  Scales as check_scales.  Where a group's scale is inexact
    because the GPU rounded the group's largest activation to the
    neighbouring dtype value (reading R14; an E8M0 step when that crosses a
    power of two), the group's codes are compared with the oracle's codes of
    its rounded row with that element moved one dtype value the same way
    (they change with the scale); every other code with the oracle's.  Then
    the code rule (equal, or one apart in at most floor(n / 1000)).
    Returns (codes one apart, inexact scales, list of inexact groups)."""
    nbad, listed = check_scales(gpu_scales, ref_scales, mode, name + ".scales", u=u, dtype=dtype,
                                allowed=allowed_scales)
    ref_codes = np.array(ref_values, dtype=np.uint8, copy=True)
    listed = list(listed)
    if listed and u is not None:
        gs = np.asarray(gpu_scales)
        rs = np.asarray(ref_scales)
        M, cols = ref_codes.shape
        groups = rs.reshape(M, -1).shape[1]
        width = cols // groups
        for n_, (i, why) in enumerate(listed):
            r, j = divmod(i, groups)
            g_val, r_val = gs.reshape(M, -1)[r, j], rs.reshape(M, -1)[r, j]
            up = bool(g_val > r_val)
            q, sc = _moved_group_quant(np.asarray(u)[r], j * width, (j + 1) * width, up, dtype, mode)
            if q is None:
                continue
            s0 = np.asarray(sc).ravel()[0]
            same = (int(s0) == int(g_val)) if mode == 0 else \
                (np.float32(s0).view(np.uint32) == np.float32(g_val).view(np.uint32))
            if same:
                ref_codes[r, j * width:(j + 1) * width] = q
                if mode == 0:
                    listed[n_] = (i, "R14: E8M0 step, amax one dtype value away")
            elif mode == 0:
                raise AssertionError(f"{name}: E8M0 step at group {i} not explained by a one-value "
                                     f"move of the group's largest activation")
    n1 = check_codes(gpu_values, ref_codes, name + ".codes", allowed=allowed_codes)
    return n1, nbad, listed


def scales_u8_or_f32(t):
    """torch scales tensor -> numpy (uint8 or float32)."""
    import torch
    a = t.detach().cpu()
    if a.dtype == torch.uint8:
        return a.numpy()
    return a.float().numpy()
