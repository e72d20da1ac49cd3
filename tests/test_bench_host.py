"""Host-side logic of bench.py (no GPU): the algorithmic flop and byte counts
its roofline figures divide by, the traffic table's tie to the kernel sources,
and the refusal of more than one GPU."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_flop_count_per_token_head():
    """The chunk algorithm as written, full 64 x 64 tiles, at d = 128: the
    prep's K K^T, Q K^T, W and u (4 x 2 C d) and the scan's W S, Q~ S, K~^T U
    (3 x 2 d^2) and attn U (2 C d)."""
    d, C = 128, 64
    assert bench.flops_prep(d) == 4 * 2 * C * d == 65536
    assert bench.flops_scan(d) == 3 * 2 * d * d + 2 * C * d == 114688
    assert bench.flops_prep(d) + bench.flops_scan(d) == 180224


def test_compulsory_bytes():
    # prefill 4x8x2048, bf16: q, k, v read, o written (4 d elements), beta and g
    # read (2), the final fp32 state written
    assert bench.bytes_prefill(4, 8, 2048, 128) == 4 * 8 * 2048 * (4 * 128 * 2 + 2 * 2) + 32 * 128 * 128 * 4
    assert bench.bytes_prefill(4, 8, 2048, 128) == 69468160
    # decode 256x16: the fp32 state read and written, q, k, v, beta, g read, o written
    assert bench.decode_bytes_per_step(256, 16, 128) == 541081600


def test_traffic_tied_to_sources(monkeypatch):
    """A traffic entry reads its calibrated bytes while the kernel sources hash
    to the value it was taken on, and None once they do not."""
    name = "decode_step_kernel"
    t = dict(bench.TRAFFIC[name])
    monkeypatch.setitem(bench.TRAFFIC, name, t)
    want = int(round((t["fetch_kib"] * bench.FETCH_SCALE + t["write_kib"] * bench.WRITE_SCALE) * 1024))
    if bench.sources_sha256(t["sources"]) == t["sha256"]:
        assert bench.traffic_bytes(name) == want
    t["sha256"] = "0" * 64
    assert bench.traffic_bytes(name) is None
    assert bench.traffic_bytes("no_such_kernel") is None


@pytest.mark.parametrize("n", [2, 8])
def test_more_than_one_gpu_refused(n):
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", str(n)],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
