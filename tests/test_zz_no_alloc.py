"""moe_layout_noalloc (the entry point that allocates nothing) against
moe_layout with a caller workspace, through the C ABI: two calls in a row on
the library's shared per-GPU scratch, the second with a smaller batch, then a
batch that needs no scratch.  Every output bit for bit, and against the
oracle."""
from __future__ import annotations

import numpy as np
import pytest
import torch

import oracle
from parity_helpers import compare_layout
from workloads import CONFIGS, PAD_MULTIPLE, PAD_NONE, make_workload

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


def _routing(case):
    name, S, K, E, R, pad_mode, pad_rows = case
    if name == "dsmoe16b":
        return make_workload(CONFIGS["dsmoe16b"], with_hidden=False).topk_idx
    rng = np.random.default_rng(9100 + S)
    p = rng.random(E) ** 2
    idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
    idx.reshape(-1)[rng.integers(0, idx.size, 9)] = E + 1          # invalid ids are flagged, not placed
    return idx


CASES = [
    # name, S, K, E, R, pad_mode, pad_rows: two-launch (scratch), smaller two-launch, one-launch
    ("dsmoe16b", 16384, 6, 64, 8, PAD_NONE, 0),
    ("N40000-E96-pad16", 5000, 8, 96, 6, PAD_MULTIPLE, 16),
    ("N4096-E256", 512, 8, 256, 8, PAD_NONE, 0),
]


def test_noalloc_matches_layout():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_02_amd as moe
    for case in CASES:
        name, S, K, E, R, pad_mode, pad_rows = case
        print(f"case noalloc {name}: S={S} K={K} E={E} R={R} pad={pad_mode}/{pad_rows}", flush=True)
        idx = _routing(case)
        desc = moe.LayoutDesc(S, K, E, R, pad_mode, pad_rows)
        idx_d = torch.from_numpy(idx).to(DEV)
        want = moe.moe_layout(desc, idx_d)                      # caller-provided workspace
        got = moe.alloc_layout(desc, DEV)
        got.workspace = None
        for t in (got.tokens_per_expert, got.tokens_per_rank, got.expert_offset, got.rank_offset, got.pos,
                  got.src, got.status):
            t.fill_(-7)
        moe.moe_layout_noalloc(desc, idx_d, got)
        torch.cuda.synchronize()
        for f in ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status"):
            assert torch.equal(getattr(got, f), getattr(want, f)), f"{name}: {f}"
        compare_layout(got, oracle.layout(idx, E, R, pad_mode, pad_rows), f"{name} noalloc")


def test_noalloc_rejects_what_does_not_fit():
    import ctypes
    import combine_moe_layout_02_amd as moe
    lib = moe.lib()
    d = moe.LayoutDesc(1 << 27, 8, 1024, 8).c()        # 2^30 entries: ~1 GB of histograms
    b = moe.moe_layout_bufs(*([1 << 20] * 7))
    assert lib.moe_layout_noalloc(ctypes.byref(d), ctypes.c_void_p(1 << 20), ctypes.byref(b), None) == \
        moe.MOE_ERR_WORKSPACE


def test_noalloc_under_graph_capture():
    """The allocation-free layout captured in a HIP graph (code under graph
    capture is a caller it exists for) and replayed with new routing written
    into the captured input between replays: every replay equals moe_layout
    (caller workspace, eager) on that routing, and the first also the oracle."""
    import combine_moe_layout_02_amd as moe
    S, K, E, R = 16384, 6, 64, 8                       # two-launch form: uses the library's scratch
    desc = moe.LayoutDesc(S, K, E, R)
    rng = np.random.default_rng(9300)

    def routing(bad: bool):
        p = rng.random(E) ** 2
        idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
        if bad:
            idx.reshape(-1)[rng.integers(0, idx.size, 11)] = -3
        return idx

    idx_d = torch.from_numpy(routing(False)).to(DEV)
    got = moe.alloc_layout(desc, DEV)
    got.workspace = None
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        moe.moe_layout_noalloc(desc, idx_d, got)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        moe.moe_layout_noalloc(desc, idx_d, got)
    torch.cuda.synchronize()
    fields = ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status")
    for rep in range(4):
        print(f"case noalloc graph replay {rep}", flush=True)
        idx = routing(bad=rep == 2)
        idx_d.copy_(torch.from_numpy(idx))
        for f in fields:
            getattr(got, f).fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        want = moe.moe_layout(desc, idx_d)
        torch.cuda.synchronize()
        for f in fields:
            assert torch.equal(getattr(got, f), getattr(want, f)), f"replay {rep}: {f}"
        if rep == 0:
            compare_layout(got, oracle.layout(idx, E, R), "noalloc graph replay")
