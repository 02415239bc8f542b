"""Hand-worked quantiser examples and the output layout stated on the pages
(tests/golden/*.txt, each carrying its derivation and citation)."""
import os

import numpy as np

import oracle as orc

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _rows(name):
    header, rows = {}, []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if not line:
                continue
            a, b = line.split()[:2]
            if a in ("scale_byte", "scale"):
                header[a] = float(b)
            else:
                rows.append((float(a), int(b, 16)))
    return header, rows


def test_mx_block_worked_example():
    hdr, rows = _rows("mx_block_worked.txt")
    u = np.zeros((1, 32), np.float32)
    for j, (v, _) in enumerate(rows):
        u[0, j] = v
    q, s = orc.quant(u, orc.FP32, orc.MXFP8)
    assert int(s[0, 0]) == int(hdr["scale_byte"])
    for j, (_, code) in enumerate(rows):
        assert q[0, j] == code, (j, hex(q[0, j]), hex(code))
    assert not q[0, len(rows):].any()


def test_fp32_scale_worked_example():
    hdr, rows = _rows("fp32_scale_worked.txt")
    u = np.zeros((1, 128), np.float32)
    for j, (v, _) in enumerate(rows):
        u[0, j] = v
    for mode in (orc.BLOCK128, orc.PER_TOKEN):
        q, s = orc.quant(u, orc.FP32, mode)
        assert float(s[0, 0]) == hdr["scale"]
        for j, (_, code) in enumerate(rows):
            assert q[0, j] == code, (mode, j, hex(q[0, j]), hex(code))
        assert not q[0, len(rows):].any()


def test_layout_shapes():
    modes = {"mxfp8": orc.MXFP8, "block128": orc.BLOCK128, "per_token": orc.PER_TOKEN}
    with open(os.path.join(GOLDEN, "layout_shapes.txt")) as f:
        for line in f:
            if line.startswith("#") or not line.strip():
                continue
            mode, M, cols, shape, dt = line.split()[:5]
            M, cols = int(M), int(cols)
            x = np.ones((M, cols), np.float32)
            q, s = orc.quant(x, orc.FP32, modes[mode])
            assert q.shape == (M, cols)
            assert "x".join(map(str, s.shape)) == shape
            assert s.dtype == np.dtype(dt)
