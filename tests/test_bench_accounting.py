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


def test_profile_summary_arithmetic(tmp_path, monkeypatch):
    """bench.py --summarize on a synthetic profiling run: counter KiB are
    scaled by the copy calibration, summed per role, and divided by the
    algorithmic bytes of the bench line."""
    import json
    import bench
    from workloads import CONFIGS

    def write_csv(path, header, rows):
        path.parent.mkdir(parents=True, exist_ok=True)
        with open(path, "w") as f:
            f.write(",".join(f'"{h}"' for h in header) + "\n")
            for r in rows:
                f.write(",".join(f'"{v}"' for v in r) + "\n")

    comb = "void moe::(anonymous namespace)::k_combine<8>(moe::CombineArgs, int)"
    disp = "void moe::(anonymous namespace)::k_dispatch_fp8<8>(moe::DispatchArgs, int)"
    lay = "moe::(anonymous namespace)::k_layout_onepass(moe::LayoutArgs)"
    hdr = ["Kernel_Name", "Counter_Name", "Counter_Value"]
    # the 1 GiB copy reads 2^19 KiB on FETCH_SIZE (factor 2) and 2^20 KiB on WRITE_SIZE (factor 1)
    write_csv(tmp_path / "calib_FETCH_SIZE" / "calib_counter_collection.csv", hdr,
              [["copy", "FETCH_SIZE", 524288.0]] * 3 + [["fill", "FETCH_SIZE", 10.0]])
    write_csv(tmp_path / "calib_WRITE_SIZE" / "calib_counter_collection.csv", hdr,
              [["copy", "WRITE_SIZE", 1048576.0]] * 3)
    cfg = CONFIGS["prefill"]
    write_csv(tmp_path / "kt_prefill" / "prefill_kernel_stats.csv", ["Name", "Calls", "AverageNs"],
              [[comb, 20, 100000.0], [disp, 20, 50000.0], [lay, 20, 8000.0], ["other", 1, 5.0]])
    for P, vals in (("FETCH_SIZE", (1000.0, 300.0, 2.0)), ("WRITE_SIZE", (100.0, 2000.0, 1.0))):
        write_csv(tmp_path / f"pmc_{P}_prefill" / "prefill_counter_collection.csv", hdr,
                  [[comb, P, vals[0]], [comb, P, vals[0] + 2], [disp, P, vals[1]], [lay, P, vals[2]]])
    alg = {"layout": 393216, "dispatch": 301334528, "combine": 528744448}
    line = {"ms_per_step": 0.16, "value": 5000.0,
            "kernels": {"bytes": alg, "dispatch_plus_combine_gbps": 5500.0}, "percentiles": None}
    (tmp_path / "bench_prefill.json").write_text(json.dumps(line) + "\n")
    traffic_file = tmp_path / "traffic.json"
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(traffic_file))
    md = bench.summarize_profiles(str(tmp_path))
    rec = json.loads(traffic_file.read_text())
    assert rec["calibration"]["fetch_factor"] == 2.0 and rec["calibration"]["write_factor"] == 1.0
    c = rec["combine/prefill"]
    # medians of two dispatches: (1000, 1002) KiB read x 2, (100, 102) KiB written x 1
    assert c["read_bytes"] == 1001 * 1024 * 2 and c["write_bytes"] == 101 * 1024
    assert c["traffic_over_algorithmic"] == round((1001 * 2048 + 101 * 1024) / alg["combine"], 4)
    assert c["kernel"] == "k_combine<8>" and c["kernel_trace_avg_us"] == 100.0
    assert rec["dispatch/prefill"]["write_bytes"] == 2000 * 1024
    assert "k_layout_onepass | layout | 8.00 |" in md
    assert f"| k_combine<8> | combine | 100.00 | {alg['combine']:,} |" in md
