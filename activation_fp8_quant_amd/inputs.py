"""Seeded synthetic inputs shaped like the pages' workloads.

This module only draws random numbers and converts them to the activation
dtype (torch's round-to-nearest-even casts); it holds none of the method's
arithmetic.  Both the tests (GPU path and oracle) and the benchmark take
their inputs from here, as host numpy arrays:

    bf16 / fp16 tensors -> uint16 bit patterns

Draw order within a workload is fixed and listed per function; normals are
drawn in float64 from numpy's PCG64 (`default_rng(seed)`), scaled, cast to
float32, then rounded to the dtype.
"""
from __future__ import annotations

import numpy as np
import torch

_TORCH = {"bf16": torch.bfloat16, "fp16": torch.float16}


def to_bits(a: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    """float array -> uint16 bit patterns of the dtype (RNE cast by torch)."""
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(_TORCH[dtype])
    return t.view(torch.int16).numpy().view(np.uint16).copy()


def bits_to_float(b: np.ndarray, dtype: str = "bf16") -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(b, dtype=np.uint16).view(np.int16)).view(_TORCH[dtype])
    return t.float().numpy()


def norm_inputs(M: int, H: int, *, seed: int, x_std: float, r_std: float | None,
                w_kind: str, w_param: float, dtype: str = "bf16",
                outlier_frac: float = 0.0, outlier_mult: float = 50.0):
    """x ~ N(0, x_std^2) [M, H]; then r ~ N(0, r_std^2) [M, H] (if r_std is not
    None); then w: 'normal' -> N(0, w_param^2), 'uniform' -> U(1 - w_param,
    1 + w_param); then (if outlier_frac) a Bernoulli(outlier_frac) mask over
    x whose entries are multiplied by outlier_mult before rounding."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, H)) * x_std
    r = rng.standard_normal((M, H)) * r_std if r_std is not None else None
    if w_kind == "normal":
        w = rng.standard_normal(H) * w_param
    elif w_kind == "uniform":
        w = rng.uniform(1.0 - w_param, 1.0 + w_param, H)
    else:
        raise ValueError(w_kind)
    if outlier_frac:
        mask = rng.random((M, H)) < outlier_frac
        x = np.where(mask, x * outlier_mult, x)
    return dict(x=to_bits(x, dtype), r=None if r is None else to_bits(r, dtype),
                w=to_bits(w, dtype))


def two_segment_inputs(M: int, widths=(1536, 512), *, seed: int, dtype: str = "bf16",
                       outlier_frac: float = 0.01, outlier_mult: float = 50.0):
    """Two row segments (q / kv of an MLA attention input): for each segment
    in order, x ~ N(0,1) with a Bernoulli(outlier_frac) x outlier_mult mask,
    then w ~ U(0.5, 1.5)."""
    rng = np.random.default_rng(seed)
    segs = []
    for n in widths:
        x = rng.standard_normal((M, n))
        mask = rng.random((M, n)) < outlier_frac
        x = np.where(mask, x * outlier_mult, x)
        w = rng.uniform(0.5, 1.5, n)
        segs.append(dict(x=to_bits(x, dtype), w=to_bits(w, dtype)))
    return segs


def gate_up_inputs(M: int, I: int, *, seed: int, std: float):
    """gate_up [M, 2I] bf16, every entry ~ N(0, std^2) (gate and up halves
    drawn together, row-major)."""
    rng = np.random.default_rng(seed)
    return to_bits(rng.standard_normal((M, 2 * I)) * std, "bf16")


def edge_rows(H: int, dtype: str = "bf16", seed: int = 7) -> np.ndarray:
    """Special rows for correctness runs ([P1] test plan: all-zero, tiny,
    dominated and partly-zero blocks), returned as floats [n, H]:
      0 all zero            1 tiny (~2^-120)          2 one dominant element
      per 32-block, the rest tiny   3 half-zero blocks  4 values that land on
      e4m3 ties after normalisation (powers of two times 1.0625)
      5 amax exactly 2^k in every block  6 amax 2^k * (1 - 2^-8)
      7 a row of one repeated constant."""
    rng = np.random.default_rng(seed)
    rows = []
    rows.append(np.zeros(H))
    rows.append(rng.standard_normal(H) * 2.0 ** -120)
    r = rng.standard_normal(H) * 2.0 ** -20
    r[::32] = rng.standard_normal(H // 32) * 10.0
    rows.append(r)
    r = rng.standard_normal(H)
    blk = np.arange(H) // 16
    r[blk % 2 == 1] = 0.0
    rows.append(r)
    r = (2.0 ** rng.integers(-4, 4, H)) * 1.0625 * np.where(rng.random(H) < 0.5, -1, 1)
    rows.append(r)
    r = rng.uniform(-1, 1, H)
    r[::32] = 2.0 ** rng.integers(-3, 3, H // 32)
    rows.append(r)
    r = rng.uniform(-0.5, 0.5, H)
    r[::32] = (2.0 ** rng.integers(-3, 3, H // 32)) * (1 - 2.0 ** -8)
    rows.append(r)
    rows.append(np.full(H, 0.7))
    return np.stack(rows)
