#!/usr/bin/env python3
"""Benchmark of the MoE expert-parallel hot path on one MI355X.

One step = moe_layout + moe_dispatch + moe_combine over one batch of synthetic
input already resident in HBM.  The default workload is the prefill shape
(S=4096 tokens, H=7168, E=256 experts in 8 groups, top-4 groups / top-8
experts, R=8 simulated ranks, FP8 E4M3 dispatch with per-128-channel fp32
scales, bf16 combine).  Prints one JSON line.

Timing: W untimed warm-up steps, then K timed steps bracketed by
torch.cuda.synchronize(); HIP events on the launch stream around every call
give per-kernel averages.  A percentile pass adds p10 / median / p90 per call
over 100 iterations (1000 for the decode call), back to back ("warm") and
after overwriting 512 MiB, twice the Infinity Cache ("cold").  Bytes are the
algorithmic bytes the path must move (padding rows excluded), GB = 1e9.
Beside the prefill batch the same-shape skewed batch (bf16 dispatch, segments
padded to 128 rows) is timed too.

  --gpus N           only N=1 exists: the EP ranks are partitions of one buffer
  --config NAME      tiny | prefill | decode | skew | dsmoe16b
  --calib-copy       run only a plain device copy of known size (for scaling
                     rocprofv3 FETCH_SIZE / WRITE_SIZE counters)
  --no-cpu-baseline  skip timing the CPU oracle
  --no-decode        skip the decode, balanced-layout and skewed-batch numbers
  --no-percentiles   skip the percentile pass and the streaming reference
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "dispatch+combine HBM GB/s (% of peak) at S=4096,H=7168,E=256,K=8; µs at S=128"
HBM_PEAK_GBPS = 8000.0          # MI355X HBM3E, 8 TB/s
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "traffic.json")
CSRC = os.path.join(ROOT, "combine_moe_layout_02_amd", "csrc")


# ---------------------------------------------------------------------------
# byte accounting
# ---------------------------------------------------------------------------

def row_bytes(H: int, fp8: bool) -> int:
    """Bytes of one dispatched row: bf16 payload, or E4M3 codes plus one fp32
    scale per 128 channels."""
    return H + 4 * (H // 128) if fp8 else 2 * H


def message_bytes(S: int, K: int, H: int, fp8: bool, combine: bool) -> int:
    """Payload bytes of one dispatch or combine, counted one message per
    (token, k) entry: the convention that reproduces the GB/s column of
    DeepEP's low-latency benchmark table from its latency column."""
    return S * K * (2 * H if combine else row_bytes(H, fp8))


def layout_bytes(S: int, K: int, max_recv: int) -> int:
    # read topk_idx, write pos, write src
    return 8 * S * K + 4 * max_recv


def dispatch_bytes(S: int, K: int, H: int, fp8: bool, placed: int) -> int:
    # read hidden once; write every placed row (+ scales); pos, weight, recv_w per entry
    return 2 * S * H + placed * row_bytes(H, fp8) + 12 * S * K


def combine_bytes(S: int, K: int, H: int, placed: int, shared: bool) -> int:
    # gather every placed row, pos + weight per entry, write out (+ read shared)
    return placed * 2 * H + 8 * S * K + 2 * S * H + (2 * S * H if shared else 0)


# ---------------------------------------------------------------------------

def sources_sha256(names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(CSRC, n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()


def load_traffic(key: str):
    """HBM bytes per launch from the committed rocprofv3 counter runs, or None
    when a source of the kernel changed since they were taken."""
    try:
        with open(TRAFFIC_FILE) as f:
            rec = json.load(f)
    except (OSError, ValueError):
        return None
    entry = rec.get(key)
    if not entry or entry.get("source_sha256") != sources_sha256(entry.get("sources", [])):
        return None
    return entry.get("bytes_per_launch")


class Run:
    """Device buffers and prepared launches of one workload."""

    def __init__(self, moe, cfg, dev, seed=None):
        import numpy as np
        import torch
        from workloads import make_workload
        self.cfg = cfg
        w = make_workload(cfg, seed=seed)
        self.w = w
        self.buf = moe.Buffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=cfg.fp8, pad_mode=cfg.pad_mode,
                              pad_rows=cfg.pad_rows, device=dev)
        self.rows = self.buf.rows
        self.idx = torch.from_numpy(w.topk_idx).to(dev)
        self.hidden = torch.from_numpy(w.hidden.view(np.int16)).to(dev).view(torch.bfloat16)
        self.topk_w = torch.from_numpy(w.topk_w).to(dev)
        self.shared = (torch.from_numpy(w.shared.view(np.int16)).to(dev).view(torch.bfloat16)
                       if w.shared is not None else None)
        # stand-in expert outputs: seeded N(0,1) bf16 for every row
        g = torch.Generator(device=dev)
        g.manual_seed(w.seed)
        self.expert_out = torch.randn((self.rows, cfg.H), generator=g, device=dev,
                                      dtype=torch.float32).to(torch.bfloat16)
        # validate every argument once; the timed calls skip the Python checks
        self.buf.layout_call(self.idx)
        self.buf.dispatch_call(self.hidden, self.idx, self.topk_w)
        self.buf.combine_call(self.expert_out, self.topk_w, self.shared)
        torch.cuda.synchronize()
        self.placed = int(self.buf.layout.tokens_per_expert.sum().item())

    def layout_call(self):
        self.buf.layout_call(self.idx, check=False)

    def dispatch_call(self):
        self.buf.dispatch_call(self.hidden, self.idx, self.topk_w, check=False)

    def combine_call(self):
        self.buf.combine_call(self.expert_out, self.topk_w, self.shared, check=False)

    def layout_dispatch_call(self):
        self.buf.layout_dispatch_call(self.hidden, self.idx, self.topk_w, check=False)

    def step(self):
        self.layout_call()
        self.dispatch_call()
        self.combine_call()

    def fused_step(self):
        self.layout_dispatch_call()
        self.combine_call()

    def bytes(self):
        c = self.cfg
        return (layout_bytes(c.S, c.K, self.rows),
                dispatch_bytes(c.S, c.K, c.H, c.fp8, self.placed),
                combine_bytes(c.S, c.K, c.H, self.placed, c.shared))


def time_steps(run, steps: int, warmup: int):
    """Two timed passes of `steps` steps after `warmup` untimed ones.
    Headline pass: HIP events only at the ends of the timed region (nothing is
    inserted between the kernels).  Breakdown pass: events around every call,
    giving per-call averages (ms) on the launch stream."""
    import torch
    for _ in range(warmup):
        run.step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    a.record()
    for _ in range(steps):
        run.step()
    b.record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    step_ms = a.elapsed_time(b) / steps

    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(steps)]
    for i in range(steps):
        ev[i][0].record()
        run.layout_call()
        ev[i][1].record()
        run.dispatch_call()
        ev[i][2].record()
        run.combine_call()
        ev[i][3].record()
    torch.cuda.synchronize()
    lay = sum(e[0].elapsed_time(e[1]) for e in ev) / steps
    dis = sum(e[1].elapsed_time(e[2]) for e in ev) / steps
    com = sum(e[2].elapsed_time(e[3]) for e in ev) / steps
    return dict(layout_ms=lay, dispatch_ms=dis, combine_ms=com, step_ms=step_ms, wall_s=wall)


def call_percentiles(calls, names, iters: int, flush_bytes: int = 0):
    """p10 / median / p90 (µs) of each call over `iters` iterations, HIP events
    on the launch stream around every call.  With flush_bytes, every iteration
    first overwrites a scratch buffer of that size (twice the 256 MB
    Infinity Cache for 512 MiB) outside the event pairs: cold-cache timing."""
    import numpy as np
    import torch
    scratch = torch.empty(flush_bytes, dtype=torch.uint8, device="cuda") if flush_bytes else None
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(len(calls) + 1)] for _ in range(iters)]
    for i in range(iters):
        if scratch is not None:
            scratch.fill_(i & 0xFF)
        ev[i][0].record()
        for j, call in enumerate(calls):
            call()
            ev[i][j + 1].record()
    torch.cuda.synchronize()
    out = {}
    for j, name in enumerate(names):
        us = np.array([ev[i][j].elapsed_time(ev[i][j + 1]) * 1e3 for i in range(iters)])
        out[name] = [round(float(x), 2) for x in np.percentile(us, [10, 50, 90])]
    del scratch
    return out


def percentile_numbers(run, drun, iters: int = 100, decode_iters: int = 1000, trun=None):
    """Per-call p10 / median / p90 of the step's kernels, warm (back to back)
    and cold (after a 512 MiB overwrite), at the batch shape, at decode and
    for the tiny batch (cache-resident: no roofline claim)."""
    big = {"calls": ["layout", "dispatch", "combine"], "iters": iters}
    calls = (run.layout_call, run.dispatch_call, run.combine_call)
    big["warm_us"] = call_percentiles(calls, big["calls"], iters)
    big["cold_us"] = call_percentiles(calls, big["calls"], iters, 512 << 20)
    res = {"unit": "us [p10, p50, p90]", "batch": big}
    if drun is not None:
        dec = {"calls": ["layout_dispatch", "combine"], "iters": decode_iters}
        dcalls = (drun.layout_dispatch_call, drun.combine_call)
        dec["warm_us"] = call_percentiles(dcalls, dec["calls"], decode_iters)
        dec["cold_us"] = call_percentiles(dcalls, dec["calls"], decode_iters, 512 << 20)
        res["decode"] = dec
    if trun is not None:
        tiny = {"calls": big["calls"], "iters": decode_iters}
        tcalls = (trun.layout_call, trun.dispatch_call, trun.combine_call)
        tiny["warm_us"] = call_percentiles(tcalls, tiny["calls"], decode_iters)
        tiny["cold_us"] = call_percentiles(tcalls, tiny["calls"], decode_iters, 512 << 20)
        res["tiny"] = tiny
    return res


def shape_numbers(moe, cfg, dev, steps: int = 30, warmup: int = 5):
    """Dispatch + combine GB/s and % of peak of another workload (the skewed
    batch has the metric's shape with bf16 dispatch and padding)."""
    r = Run(moe, cfg, dev)
    _, db, cb = r.bytes()
    t = time_steps(r, steps, warmup)
    dc = (db + cb) / ((t["dispatch_ms"] + t["combine_ms"]) * 1e-3) / 1e9
    out = {"workload": cfg.name, "fp8_dispatch": cfg.fp8, "pad_mode": cfg.pad_mode, "pad_rows": cfg.pad_rows,
           "dispatch_us": round(t["dispatch_ms"] * 1e3, 2), "combine_us": round(t["combine_ms"] * 1e3, 2),
           "layout_us": round(t["layout_ms"] * 1e3, 2), "dispatch_plus_combine_gbps": round(dc, 1),
           "dispatch_plus_combine_frac_of_peak": round(dc / HBM_PEAK_GBPS, 4),
           "bytes": {"dispatch": db, "combine": cb}}
    del r
    return out


def streaming_reference(cfg, dev, iters: int = 50):
    """What a plain streaming kernel reaches at combine's byte mix on this GPU
    in this process: torch.sum over K contiguous bf16 planes of S*H into one
    (the same bytes in and out as combine, with no gather)."""
    import torch
    x = torch.empty((cfg.K, cfg.S * cfg.H), dtype=torch.bfloat16, device=dev).normal_()
    out = torch.empty(cfg.S * cfg.H, dtype=torch.bfloat16, device=dev)
    ms = time_calls(lambda: torch.sum(x, dim=0, out=out), iters, 10)
    nbytes = (cfg.K + 1) * cfg.S * cfg.H * 2
    del x, out
    return {"what": f"torch.sum of {cfg.K} contiguous bf16 planes [{cfg.S}x{cfg.H}] into one (same bytes as "
                    "combine, no gather)", "gbps": round(nbytes / (ms * 1e-3) / 1e9, 1)}


def time_graph(step, iters: int, calls_per_graph: int = 1):
    """`calls_per_graph` steps captured once in a HIP graph, replayed `iters`
    times; returns ms per step."""
    import torch
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(calls_per_graph):
            step()
    for _ in range(10):
        graph.replay()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        graph.replay()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / (iters * calls_per_graph)


def time_calls(step, iters: int, warmup: int = 20):
    """Average ms per step, events only at the ends of the timed region."""
    import torch
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(iters):
        step()
    b.record()
    torch.cuda.synchronize()
    return a.elapsed_time(b) / iters


def decode_numbers(moe, dcfg, dev, iters: int, drun=None):
    """µs per decode call (S=128): moe_layout_dispatch (one launch) + moe_combine,
    eager and graph-replayed, and the three-call variant."""
    drun = drun if drun is not None else Run(moe, dcfg, dev)
    dt = time_steps(drun, iters, 20)
    fused_ms = time_calls(drun.fused_step, iters)
    ld_ms = time_calls(drun.layout_dispatch_call, iters)
    comb_ms = time_calls(drun.combine_call, iters)
    g_ms = time_graph(drun.fused_step, iters)
    # a model's decode step captures every layer's calls in one graph: per
    # call inside a 64-call graph (64 MoE layers' dispatch + combine)
    g64_ms = time_graph(drun.fused_step, max(iters // 64, 4), 64)
    return {"us_per_call": round(fused_ms * 1e3, 2),
            "call": "moe_layout_dispatch (one launch) + moe_combine",
            "layout_dispatch_us": round(ld_ms * 1e3, 2), "combine_us": round(comb_ms * 1e3, 2),
            "graph_replay_us_per_call": round(g_ms * 1e3, 2),
            "graph_of_64_calls_us_per_call": round(g64_ms * 1e3, 2),
            "three_call_us_per_call": round(dt["step_ms"] * 1e3, 2),
            "config": {"workload": "decode", "S": dcfg.S, "H": dcfg.H, "E": dcfg.E, "K": dcfg.K,
                       "R": dcfg.R, "fp8": dcfg.fp8, "capacity": dcfg.pad_rows}}


def cu_budget_numbers(moe, run, counts, steps: int = 10):
    """Dispatch + combine GB/s when the step runs on a stream limited to n CUs."""
    import torch
    out = {}
    _, db, cb = run.bytes()
    for n in counts:
        with moe.CULimitedStream(n) as cs:
            with torch.cuda.stream(cs.stream):
                t = time_steps(run, steps, 3)
            torch.cuda.synchronize()
        out[str(n)] = {"dispatch_plus_combine_gbps": round((db + cb) / ((t["dispatch_ms"] + t["combine_ms"]) * 1e-3) / 1e9, 1),
                       "step_us": round(t["step_ms"] * 1e3, 1)}
    return out


def overlap_numbers(moe, run, dev, steps: int = 10, gemms: int = 4):
    """The step on one half of the CUs while a bf16 GEMM of the layer's shape
    ([S,H] x [H,H]) runs on the other half: each alone, then both at once."""
    import torch
    n_cu = torch.cuda.get_device_properties(dev).multi_processor_count
    half = n_cu // 2
    cfg = run.cfg
    a = torch.randn(cfg.S, cfg.H, device=dev, dtype=torch.float32).to(torch.bfloat16)
    b = torch.randn(cfg.H, cfg.H, device=dev, dtype=torch.float32).to(torch.bfloat16)
    c = torch.empty(cfg.S, cfg.H, device=dev, dtype=torch.bfloat16)
    _, db, cb = run.bytes()
    with moe.CULimitedStream(half, dev, first_cu=0) as sa, moe.CULimitedStream(half, dev, first_cu=half) as sb:
        def on_a():
            for _ in range(steps):
                run.step()

        def on_b():
            for _ in range(gemms):
                torch.matmul(a, b, out=c)

        def timed(work):   # list of (stream, fn): ms per stream, and the whole span
            torch.cuda.synchronize()
            ev = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in work]
            t0 = time.perf_counter()
            for (st, fn), (e0, e1) in zip(work, ev):
                with torch.cuda.stream(st):
                    e0.record()
                    fn()
                    e1.record()
            torch.cuda.synchronize()
            wall = (time.perf_counter() - t0) * 1e3
            return [e0.elapsed_time(e1) for e0, e1 in ev], wall

        for st, fn in ((sa.stream, on_a), (sb.stream, on_b)):   # warm-up
            with torch.cuda.stream(st):
                fn()
        (t_a,), _ = timed([(sa.stream, on_a)])
        (t_b,), _ = timed([(sb.stream, on_b)])
        (ta2, tb2), wall = timed([(sa.stream, on_a), (sb.stream, on_b)])
    del a, b, c
    flops = 2.0 * cfg.S * cfg.H * cfg.H * gemms
    return {"cus_each": half, "steps": steps, "gemm": f"{gemms} x bf16 [{cfg.S}x{cfg.H}] x [{cfg.H}x{cfg.H}]",
            "step_alone_us": round(t_a / steps * 1e3, 1), "gemm_alone_us": round(t_b / gemms * 1e3, 1),
            "step_overlapped_us": round(ta2 / steps * 1e3, 1), "gemm_overlapped_us": round(tb2 / gemms * 1e3, 1),
            "dispatch_plus_combine_gbps_overlapped": round((db + cb) * steps / (ta2 * 1e-3) / 1e9, 1),
            "gemm_tflops_alone": round(flops / (t_b * 1e-3) / 1e12, 1),
            "gemm_tflops_overlapped": round(flops / (tb2 * 1e-3) / 1e12, 1),
            "sum_alone_over_both_wall": round((t_a + t_b) / wall, 3)}


def balanced_numbers(moe, cfg, dev, slots: int = 16, iters: int = 200):
    """Balanced layout (redundant-expert slots) on a skewed batch: time per
    call next to the plain layout, and rows per rank before / after."""
    import numpy as np
    import torch
    from workloads import make_workload
    w = make_workload(cfg, with_hidden=False)
    desc = moe.LayoutDesc(cfg.S, cfg.K, cfg.E, cfg.R)
    idx = torch.from_numpy(w.topk_idx).to(dev)
    lay = moe.alloc_layout(desc, dev)
    bal = moe.alloc_balance(desc, slots, dev)
    moe.moe_layout(desc, idx, lay)
    torch.cuda.synchronize()
    plain_rows = lay.tokens_per_rank.cpu().numpy()
    plain_ms = time_calls(lambda: moe.moe_layout(desc, idx, lay), iters)
    bal_ms = time_calls(lambda: moe.moe_layout_balanced(desc, slots, idx, lay, bal), iters)
    rows = lay.tokens_per_rank.cpu().numpy()
    status = int(lay.status.cpu().numpy()[0])
    used = int((bal.slot_expert.cpu().numpy()[:cfg.R * slots] >= 0).sum())
    return {"workload": cfg.name, "slots_per_rank": slots, "balanced_layout_us": round(bal_ms * 1e3, 2),
            "plain_layout_us": round(plain_ms * 1e3, 2),
            "rows_per_rank_max_over_mean_plain": round(float(plain_rows.max() / plain_rows.mean()), 3),
            "rows_per_rank_max_over_mean_balanced": round(float(rows.max() / rows.mean()), 3),
            "replica_slots_used": used, "unbalanced_flag": bool(status & 4)}


def cpu_baseline(cfg, budget_s: float = 12.0):
    """The CPU oracle (single-threaded C) on the same workload: layout, dispatch
    and combine of full batches, repeated until ~budget_s of work."""
    import numpy as np
    import oracle
    from workloads import make_workload, random_expert_out_bits
    w = make_workload(cfg)
    rows = oracle.max_recv_rows(cfg.S, cfg.K, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    y = random_expert_out_bits(w.seed, rows, cfg.H)
    # one core: the oracle is single-threaded; pin it so the figure is per core
    old_aff = os.sched_getaffinity(0) if hasattr(os, "sched_getaffinity") else None
    if old_aff:
        os.sched_setaffinity(0, {min(old_aff)})
    passes, t_total, nbytes, times = 0, 0.0, 0, []
    while t_total < budget_s or passes == 0:
        t0 = time.perf_counter()
        lo = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
        if cfg.fp8:
            oracle.dispatch_fp8(w.hidden, lo.pos, rows, w.topk_w)
        else:
            oracle.dispatch_bf16(w.hidden, lo.pos, rows, w.topk_w)
        oracle.combine(y, lo.pos, w.topk_w, w.shared)
        times.append(time.perf_counter() - t0)
        t_total += times[-1]
        passes += 1
        placed = int(lo.tokens_per_expert.sum())
        nbytes += (layout_bytes(cfg.S, cfg.K, rows) + dispatch_bytes(cfg.S, cfg.K, cfg.H, cfg.fp8, placed)
                   + combine_bytes(cfg.S, cfg.K, cfg.H, placed, cfg.shared))
        del lo
    if old_aff:
        os.sched_setaffinity(0, old_aff)
    return {"value": round(nbytes / t_total / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{passes} full {cfg.name} batches (S={cfg.S}, layout + "
                      f"{'fp8' if cfg.fp8 else 'bf16'} dispatch + combine), {t_total:.1f} s single-threaded",
            "ms_per_step": round(1e3 * t_total / passes, 2),
            "ms_per_step_median": round(1e3 * float(np.median(times)), 2), "host_cpus": os.cpu_count(),
            "cpu_model": cpu_model(), "pinned_core": min(old_aff) if old_aff else None}


def cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def calib_copy(nbytes: int = 1 << 30):
    """A plain device-to-device copy of a known size, for counter scaling."""
    import torch
    a = torch.empty(nbytes // 4, dtype=torch.float32, device="cuda:0").fill_(1.0)
    b = torch.empty_like(a)
    for _ in range(3):
        b.copy_(a)
    torch.cuda.synchronize()
    print(json.dumps({"calib_copy_bytes": nbytes, "launches": 3}))


def main(argv=None):
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="prefill")
    ap.add_argument("--decode-iters", type=int, default=500)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-decode", action="store_true")
    ap.add_argument("--cu-budgets", default="32,64,128,256",
                    help="comma-separated CU counts for the CU-limited-stream sweep ('' to skip)")
    ap.add_argument("--calib-copy", action="store_true")
    ap.add_argument("--only-decode", action="store_true",
                    help="time only the decode call (S=128) and print its JSON object")
    ap.add_argument("--no-percentiles", action="store_true",
                    help="skip the per-call p10/p50/p90 pass (warm and after a 512 MiB cache flush) "
                         "and the streaming reference")
    ap.add_argument("--only-balanced", action="store_true",
                    help="time only the balanced layout on the skew batch and print its JSON object")
    args = ap.parse_args(argv)

    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU: the EP ranks are simulated as partitions of one HBM buffer, "
              "so --gpus must be 1", file=sys.stderr)
        sys.exit(2)
    if args.calib_copy:
        calib_copy()
        return

    import torch
    import combine_moe_layout_02_amd as moe
    from workloads import CONFIGS

    dev = torch.device("cuda:0")
    if args.only_decode:
        print(json.dumps(decode_numbers(moe, CONFIGS["decode"], dev, args.decode_iters)), flush=True)
        return
    if args.only_balanced:
        print(json.dumps(balanced_numbers(moe, CONFIGS["skew"], dev)), flush=True)
        return
    cfg = CONFIGS[args.config]
    run = Run(moe, cfg, dev)
    lb, db, cb = run.bytes()
    t = time_steps(run, args.steps, args.warmup)
    step_bytes = lb + db + cb
    value = step_bytes / (t["step_ms"] * 1e-3) / 1e9
    d_gbps = db / (t["dispatch_ms"] * 1e-3) / 1e9
    c_gbps = cb / (t["combine_ms"] * 1e-3) / 1e9
    dc_gbps = (db + cb) / ((t["dispatch_ms"] + t["combine_ms"]) * 1e-3) / 1e9

    # dominant kernel: the larger byte mover of dispatch and combine
    dom = "combine" if cb >= db else "dispatch"
    dom_bytes, dom_ms = (cb, t["combine_ms"]) if dom == "combine" else (db, t["dispatch_ms"])
    achieved = dom_bytes / (dom_ms * 1e-3) / 1e9
    roofline = {"bound": "hbm", "achieved": round(achieved, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                "frac": round(achieved / HBM_PEAK_GBPS, 4), "traffic": load_traffic(f"{dom}/{cfg.name}"),
                "traffic_unit": "HBM bytes per launch",
                "kernel": dom, "algorithmic_bytes_per_launch": dom_bytes,
                "avg_launch_us": round(dom_ms * 1e3, 2)}
    if dom == "combine" and not args.no_percentiles:
        ref = streaming_reference(cfg, dev)
        ref["kernel_over_reference"] = round(achieved / ref["gbps"], 3)
        roofline["streaming_reference"] = ref

    extra = {"layout_us": round(t["layout_ms"] * 1e3, 2), "dispatch_us": round(t["dispatch_ms"] * 1e3, 2),
             "combine_us": round(t["combine_ms"] * 1e3, 2), "dispatch_gbps": round(d_gbps, 1),
             "combine_gbps": round(c_gbps, 1), "dispatch_plus_combine_gbps": round(dc_gbps, 1),
             "dispatch_plus_combine_frac_of_peak": round(dc_gbps / HBM_PEAK_GBPS, 4),
             "bytes": {"layout": lb, "dispatch": db, "combine": cb}, "wall_s_timed": round(t["wall_s"], 3)}

    drun = None if args.no_decode else Run(moe, CONFIGS["decode"], dev)
    decode = None if args.no_decode else decode_numbers(moe, CONFIGS["decode"], dev, args.decode_iters, drun)
    pct = None if args.no_percentiles else percentile_numbers(
        run, drun, trun=None if args.no_decode else Run(moe, CONFIGS["tiny"], dev))
    also = None
    if not args.no_decode and cfg.name == "prefill":
        also = shape_numbers(moe, CONFIGS["skew"], dev)
    balanced = None if args.no_decode else balanced_numbers(moe, CONFIGS["skew"], dev)
    budgets = [int(x) for x in args.cu_budgets.split(",") if x.strip()]
    cu_budget = cu_budget_numbers(moe, run, budgets) if budgets else None
    overlap = overlap_numbers(moe, run, dev) if budgets else None

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cfg)

    line = {
        "metric": METRIC, "value": round(value, 1), "unit": "GB/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(t["step_ms"], 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "f32", "data": "synthetic",
        "config": {"workload": cfg.name, "S": cfg.S, "H": cfg.H, "E": cfg.E, "K": cfg.K, "R": cfg.R,
                   "fp8_dispatch": cfg.fp8, "routing": cfg.routing, "pad_mode": cfg.pad_mode,
                   "pad_rows": cfg.pad_rows, "shared": cfg.shared, "parallelism": f"ep{cfg.R} simulated on 1 GPU"},
        "roofline": roofline, "cpu_baseline": cpu, "kernels": extra, "decode": decode,
        "cu_budget": cu_budget, "overlap": overlap, "balanced_layout": balanced, "percentiles": pct, "same_shape_skew": also,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
