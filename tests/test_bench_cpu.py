"""Host-side checks of bench.py: the one-GPU rule and the roofline arithmetic."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402


def test_more_than_one_gpu_exits_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"] and msg["gpus_requested"] == 2


def test_scan_flop_counts_are_ordered_and_match_hand_counts():
    T, H, d, c = 8192, 48, 128, 64
    alg = bench.scan_algorithmic_flops(T, H)
    passes = bench.scan_pass_flops(T, H)
    issued = bench.scan_issued_flops(T, H)
    # per token and head: three d x d products (2 d^2 each) and two half 64 x 64 products
    assert alg == T * H * (3 * 2 * d * d + 2 * c * d)
    assert alg < passes < issued
    # issued: 150 MFMAs of 16x16x32 per 16-row slab and chunk
    assert issued == (T // c) * H * (d // 16) * 150 * 16384


def test_flush_bytes_count_each_touched_state_twice_and_rows_once():
    state = 32 * 128 * 128 * 4
    row = 16 * 128 * 2 + 32 * 128 * 2 + 2 * 32 * 4
    assert bench.flush_bytes([0, 0]) == 0
    assert bench.flush_bytes([1, 3]) == 2 * (2 * state) + 4 * row
