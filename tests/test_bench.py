"""Host-side checks of the benchmark's accounting (no GPU)."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_flops_formula():
    # 4 B H N^2 d for the forward, halved under the causal mask; backward 2.5x
    f, b = bench.flops(2, 8192, 16, 128, True)
    assert f == 4.0 * 2 * 16 * 8192 ** 2 * 128 / 2
    assert b == 2.5 * f
    f, _ = bench.flops(1, 100, 3, 64, False)
    assert f == 4.0 * 100 ** 2 * 3 * 64


def _pairs_brute(N, bq, bc, causal):
    # (query tile, key tile) pairs holding at least one visible (query, key)
    n = 0
    for i in range(0, N, bq):
        for j in range(0, N, bc):
            qs, ks = range(i, min(i + bq, N)), range(j, min(j + bc, N))
            if not causal or any(k <= q for q in qs for k in ks):
                n += 1
    return n


def test_dq_reduction_bytes_counts_visible_tile_pairs():
    for N, d, causal in ((1000, 128, True), (777, 64, False), (600, 256, True), (300, 256, False)):
        bc = 128 if d == 256 else 256
        want = _pairs_brute(N, 32, bc, causal) * 2 * 3 * 32 * d * 4
        assert bench.dq_reduction_bytes(2, N, 3, d, causal) == want
    # the headline workload: 4224 pairs per head, 32 heads, 16 KiB per pair
    assert bench.dq_reduction_bytes(2, 8192, 16, 128, True) == 4224 * 32 * 16384


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_code_only_drops_comments_and_blank_lines():
    src = "int a;  // note\n\n/* block\n comment */ int b;\nconst char* s = 0;\n"
    assert bench.code_only(src) == "int a;\n int b;\nconst char* s = 0;"
