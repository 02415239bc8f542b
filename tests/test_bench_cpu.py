"""bench.py on the host: the refusal of more than one GPU, and the byte
formulas that the reported rates and the roofline's achieved bandwidth rest
on, against sums written out from the buffers each launch reads and writes
(include/afq.h: codes 1 byte per element, E8M0 scales 1 byte per 32, fp32
scales 4 bytes per 128 elements or per row)."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402  (imports no GPU code at module level)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_headline_bytes():
    # add + Gemma RMSNorm + MXFP8 + bf16 copy, M = 16384, H = 6144 (bf16):
    # read x and r, write h, the copy, the codes and the E8M0 scales; the
    # weight once
    M, H = 16384, 6144
    per_row = 2 * H + 2 * H + 2 * H + 2 * H + H + H // 32
    assert bench.norm_bytes(M, H) == M * per_row + 2 * H == 909_127_680


def test_other_workload_bytes():
    # 1x128 norm without copy, H = 4096, M = 4096: x, r, h, codes, fp32 scales
    assert bench.norm_bytes(4096, 4096, normed=False, mode="b128") == \
        4096 * (3 * 2 * 4096 + 4096 + 4 * 32) + 2 * 4096
    # SiLU-and-mul, 1x128, I = 12288, M = 4096: [gate | up] bf16 in, codes and fp32 scales out
    assert bench.silu_bytes(4096, 12288, mode="b128") == 4096 * (2 * 2 * 12288 + 12288 + 4 * 96)
    # MXFP8, I = 768: 24 E8M0 bytes per row
    assert bench.silu_bytes(8, 768) == 8 * (4 * 768 + 768 + 24)
    # two per-token segments of 1536 and 512, no residual, no copy: x, codes, one fp32 scale
    # per row per segment, both weights once
    assert bench.two_seg_bytes(8192) == 8192 * (3 * 2048 + 2 * 4) + 2 * 2048


def test_committed_traffic_record_uses_the_same_bytes():
    with open(os.path.join(ROOT, "profiles", "traffic_norm_mx_h6144_m16384.json")) as fh:
        rec = json.load(fh)
    assert rec["algorithmic_bytes_per_launch"] == bench.norm_bytes(16384, 6144)
    ratio = rec["traffic_bytes_per_launch"] / rec["algorithmic_bytes_per_launch"]
    assert 0.99 < ratio < 1.05, ratio


def test_copy_only_bytes():
    # the copy-only launches (the in-repo memory-pattern figures): the norm
    # reads x and r and writes h and the rounded copy; the weight once
    assert bench.norm_bytes(4096, 6144, quant=False) == 4096 * 4 * 2 * 6144 + 2 * 6144
    assert bench.norm_bytes(4096, 4096, mode="b128", quant=False) == 4096 * 4 * 2 * 4096 + 2 * 4096
    # SiLU-and-mul: [gate | up] in, the bf16 activation out
    assert bench.silu_bytes(16384, 3072, quant=False) == 16384 * (2 * 2 * 3072 + 2 * 3072)
    # two segments without residual: x in, the copy out, both weights once
    assert bench.two_seg_bytes(8192, quant=False) == 8192 * 2 * 2 * 2048 + 2 * 2048


def test_source_hash_ignores_comments_only():
    """The hash that ties stored counter figures to the norm kernel's
    sources sees code, not comments or layout."""
    import bench
    a = "int f(int x) { // one\n  return x + 1; /* two\n lines */ }\n"
    b = "int f(int x) {\n\n    return x + 1;   }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)
