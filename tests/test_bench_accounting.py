"""Byte accounting of bench.py, pinned to the pages and to exact counts.

The DeepEP low-latency table prints latency and bandwidth side by side; its
bandwidth column follows from the latency only under one byte convention:
one message per (token, k) entry carrying the FP8 row plus one fp32 scale per
128 channels for dispatch, the bf16 row for combine, GB = 1e9, truncated.
bench.py counts bytes the same way.
"""
import json
import math
import os
import subprocess
import sys

import pytest

import bench

HERE = os.path.dirname(os.path.abspath(__file__))


def table():
    with open(os.path.join(HERE, "golden", "deepep_low_latency_table.json")) as f:
        return json.load(f)


def test_low_latency_table_reproduced():
    t = table()
    S, H, K = t["S"], t["H"], t["K"]
    d = bench.message_bytes(S, K, H, fp8=True, combine=False)
    c = bench.message_bytes(S, K, H, fp8=True, combine=True)
    assert d == 128 * 8 * (7168 + 56 * 4)
    for row in t["rows"]:
        assert math.floor(d / (row["dispatch_us"] * 1e-6) / 1e9) == row["dispatch_gbps"], row
        assert math.floor(c / (row["combine_us"] * 1e-6) / 1e9) == row["combine_gbps"], row


@pytest.mark.parametrize("payload", [7168, 7168 + 56 * 2, 7168 + 112 * 4])
def test_other_conventions_do_not_fit(payload):
    """No scales, bf16 scales, or fp32 scales per 64 channels miss the table."""
    t = table()
    d = t["S"] * t["K"] * payload
    fits = [math.floor(d / (r["dispatch_us"] * 1e-6) / 1e9) == r["dispatch_gbps"] for r in t["rows"]]
    assert not all(fits)


def test_algorithmic_bytes_of_the_configs():
    # prefill: 32,768 placed rows, FP8
    assert bench.dispatch_bytes(4096, 8, 7168, True, 32768) == 301_334_528
    assert bench.combine_bytes(4096, 8, 7168, 32768, False) == 528_744_448
    # decode: 1,024 placed rows in a 32,768-row buffer
    assert bench.dispatch_bytes(128, 8, 7168, True, 1024) == 9_416_704
    assert bench.combine_bytes(128, 8, 7168, 1024, False) == 16_523_264
    assert bench.layout_bytes(128, 8, 32768) == 8 * 1024 + 4 * 32768
    # dsmoe16b: bf16 dispatch, shared output read by combine
    assert bench.dispatch_bytes(16384, 6, 2048, False, 98304) == 470_941_696
    assert bench.combine_bytes(16384, 6, 2048, 98304, True) == 537_657_344


def test_bench_refuses_more_than_one_gpu():
    r = subprocess.run([sys.executable, os.path.join(os.path.dirname(HERE), "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
