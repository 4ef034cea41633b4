"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Bar: layout, maps, counts, offsets, bf16 dispatch, FP8 codes and scales are
bit-exact; combine is within 1 bf16 ulp per element with max abs error
<= 1e-2 * max |out|.  Every input comes from the seeded generators in
`workloads`; every expected value from `oracle` on the same inputs.
Padding rows of the receive buffer are pre-filled with a NaN pattern: they
must stay untouched by dispatch and unread by combine.
"""
from __future__ import annotations

import ctypes

import numpy as np
import pytest
import torch

import oracle
from parity_helpers import (POISON_BF16, POISON_U8, assert_combine_matches, compare_layout, dev_bf16,
                            host_bits)
from workloads import (CONFIGS, PAD_CAPACITY, PAD_MULTIPLE, PAD_NONE, WorkloadConfig, make_workload,
                       random_expert_out_bits)

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def moe():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import combine_moe_layout_02_amd as m
    return m


def say(msg: str):
    print(msg, flush=True)


def run_and_check(moe, cfg: WorkloadConfig, topk_idx: np.ndarray, hidden: np.ndarray, topk_w: np.ndarray,
                  shared=None, fp8=False, seed=1, combine_weights=True):
    """Full path on the GPU vs the oracle.  Returns the oracle layout."""
    S, K, E, R, H = cfg.S, cfg.K, cfg.E, cfg.R, cfg.H
    say(f"case {cfg.name}: S={S} H={H} E={E} K={K} R={R} pad={cfg.pad_mode}/{cfg.pad_rows} fp8={fp8}")
    desc = moe.LayoutDesc(S, K, E, R, cfg.pad_mode, cfg.pad_rows)
    rows = moe.moe_max_recv_rows(desc)
    ref = oracle.layout(topk_idx, E, R, cfg.pad_mode, cfg.pad_rows)
    assert rows == len(ref.src)

    idx_d = torch.from_numpy(np.ascontiguousarray(topk_idx)).to(DEV)
    hid_d = dev_bf16(hidden, DEV)
    w_d = torch.from_numpy(np.ascontiguousarray(topk_w)).to(DEV)
    lay = moe.moe_layout(desc, idx_d)
    torch.cuda.synchronize()
    compare_layout(lay, ref, f"{cfg.name} layout")

    valid = ref.src >= 0
    if fp8:
        recv = torch.full((rows, H), POISON_U8, dtype=torch.uint8, device=DEV)
        scales = torch.full((rows, H // 128), float("nan"), dtype=torch.float32, device=DEV)
        recv_w = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_dispatch(desc, lay, hid_d, idx_d, w_d, fp8=True, recv=recv, recv_scales=scales, recv_w=recv_w)
        torch.cuda.synchronize()
        rc, rs, rw = oracle.dispatch_fp8(hidden, ref.pos, rows, topk_w)
        got_c, got_s = recv.cpu().numpy(), scales.cpu().numpy()
        bad = np.nonzero(np.any(got_c[valid] != rc[valid], axis=1))[0]
        assert bad.size == 0, f"fp8 codes differ in {bad.size} rows"
        assert np.array_equal(got_s[valid].view(np.uint32), rs[valid].view(np.uint32)), "fp8 scales differ"
        assert np.all(got_c[~valid] == POISON_U8), "dispatch wrote a padding row"
        y_ref = oracle.dequant_identity_expert(rc, rs)
    else:
        recv = torch.full((rows, H), POISON_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        recv_w = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_dispatch(desc, lay, hid_d, idx_d, w_d, fp8=False, recv=recv, recv_w=recv_w)
        torch.cuda.synchronize()
        rb, rw = oracle.dispatch_bf16(hidden, ref.pos, rows, topk_w)
        got = host_bits(recv)
        bad = np.nonzero(np.any(got[valid] != rb[valid], axis=1))[0]
        assert bad.size == 0, f"bf16 rows differ in {bad.size} rows"
        assert np.all(got[~valid] == POISON_BF16), "dispatch wrote a padding row"
        y_ref = rb
    assert np.array_equal(recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))

    w_comb = topk_w if combine_weights else None
    wc_d = w_d if combine_weights else None
    sh_d = dev_bf16(shared, DEV) if shared is not None else None
    # identity experts: the oracle's own dispatch output (dequantised for FP8)
    y = np.where(valid[:, None], y_ref, np.uint16(POISON_BF16)).astype(np.uint16)
    out = moe.moe_combine(desc, lay, dev_bf16(y, DEV), wc_d, sh_d)
    torch.cuda.synchronize()
    nx = assert_combine_matches(host_bits(out), oracle.combine(y, ref.pos, w_comb, shared), "combine/identity")
    # random expert outputs
    y = random_expert_out_bits(seed, rows, H, row_mask=valid, poison=POISON_BF16)
    out = moe.moe_combine(desc, lay, dev_bf16(y, DEV), wc_d, sh_d)
    torch.cuda.synchronize()
    nr = assert_combine_matches(host_bits(out), oracle.combine(y, ref.pos, w_comb, shared), "combine/random")
    say(f"  ok (combine elements not bit-identical: identity {nx}, random {nr})")
    return ref


@pytest.mark.parametrize("name", list(CONFIGS))
def test_config_parity(moe, name):
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    run_and_check(moe, cfg, w.topk_idx, w.hidden, w.topk_w, shared=w.shared, fp8=cfg.fp8, seed=w.seed)


def _case(name, S, H, E, K, R, pad_mode=PAD_NONE, pad_rows=0, routing="uniform"):
    return WorkloadConfig(name, S=S, H=H, E=E, K=K, R=R, pad_mode=pad_mode, pad_rows=pad_rows, routing=routing)


EDGE = [
    # (config, fp8, routing override, shared)
    (_case("one-entry", 1, 8, 1, 1, 1), False, None, False),
    (_case("ragged-row", 333, 136, 16, 16, 4), False, None, True),          # K = E, 17 vectors per row
    (_case("E1024-fp8-mult7", 777, 256, 1024, 3, 8, PAD_MULTIPLE, 7), True, None, False),
    (_case("multi-ragged-tail", 16385, 8, 5, 1, 5), False, None, False),    # one entry past one workgroup
    (_case("multi-capacity-overflow", 5000, 1024, 256, 4, 8, PAD_CAPACITY, 90), False, None, False),
    (_case("one-hot-expert", 3000, 64, 64, 1, 4, PAD_MULTIPLE, 128), False, "all5", False),
    (_case("bad-ids-fused", 100, 128, 32, 4, 4), True, "bad", False),
    (_case("bad-ids-multi", 6000, 64, 32, 4, 4, PAD_MULTIPLE, 3), False, "bad", True),
    (_case("duplicates", 300, 72, 8, 6, 2, PAD_CAPACITY, 300), False, "dup", False),
    (_case("multi-zipf", 8192, 64, 256, 8, 8, PAD_MULTIPLE, 128), False, "zipf", False),
    (_case("multi-K16-E1024", 2048, 128, 1024, 16, 1), True, None, False),
    (_case("pad-multiple-1", 50, 8, 4, 2, 2, PAD_MULTIPLE, 1), False, None, False),
    # largest layout tiles (S*K > 262144 -> 4096-entry tiles), non-power-of-two E
    (_case("tiles-4096-E96-R3", 37500, 8, 96, 8, 3, PAD_MULTIPLE, 5), False, None, False),
    # 2048-entry tiles with a capacity that some experts exceed
    (_case("tiles-2048-capacity", 20000, 16, 40, 5, 5, PAD_CAPACITY, 2500), False, None, False),
    # boundaries of the small-batch layout (S*K <= 4096 and more than 64 experts)
    (_case("small-E65-N4096", 4096, 64, 65, 1, 5), False, None, False),
    (_case("single-E64-N2048", 256, 64, 64, 8, 8), False, None, False),
    (_case("onepass-N4097-E128", 4097, 64, 128, 1, 8, PAD_MULTIPLE, 3), False, None, False),
    (_case("small-capacity-overflow", 400, 128, 128, 8, 8, PAD_CAPACITY, 20), True, None, False),
    (_case("small-bad-ids", 200, 64, 96, 4, 4, PAD_MULTIPLE, 16), False, "bad", True),
    # wide rows: many 1 KiB chunks per token, a ragged last chunk, 128 KiB
    # output rows (combine stores through a descriptor based at each row)
    (_case("wide-row-bf16-H65544", 40, 65544, 16, 4, 4), False, None, True),
    (_case("wide-row-fp8-H32896", 24, 32896, 8, 3, 2, PAD_MULTIPLE, 4), True, None, False),
]


def _random_shapes(n=40, seed=4242):
    """Seeded random shapes spanning every layout variant (single workgroup,
    one launch over tiles, two launches with 1024/2048-entry tiles), both
    dispatch formats, all pad modes and odd sizes."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = bool(rng.integers(0, 2))
        H = int(rng.integers(1, 9)) * 128 if fp8 else int(rng.integers(1, 97)) * 8
        R = int(rng.choice([1, 2, 3, 4, 5, 8, 16]))
        E = R * int(rng.integers(1, max(2, 1024 // R // 4)))
        K = int(rng.integers(1, min(16, E) + 1))
        N = int(rng.choice([rng.integers(1, 2049), rng.integers(2049, 32769), rng.integers(32769, 140000)]))
        S = max(1, N // K)
        pad = int(rng.integers(0, 3))
        pad_rows = {PAD_NONE: 0, PAD_MULTIPLE: int(rng.integers(1, 130)),
                    PAD_CAPACITY: int(max(1, S * K // E * rng.uniform(0.5, 1.5)))}[pad]
        shared = bool(rng.integers(0, 4) == 0)
        out.append((_case(f"rand{i}", S, H, E, K, R, pad, pad_rows), fp8, shared))
    return out


RANDOM_SHAPES = _random_shapes()


@pytest.mark.parametrize("case", RANDOM_SHAPES, ids=[c[0].name for c in RANDOM_SHAPES])
def test_random_shapes(moe, case):
    cfg, fp8, shared = case
    w = make_workload(cfg, seed=9000 + RANDOM_SHAPES.index(case))
    sh = make_workload(cfg, seed=9500 + RANDOM_SHAPES.index(case)).hidden if shared else None
    run_and_check(moe, cfg, w.topk_idx, w.hidden, w.topk_w, shared=sh, fp8=fp8, seed=w.seed)


@pytest.mark.parametrize("case", EDGE, ids=[c[0].name for c in EDGE])
def test_edge_cases(moe, case):
    cfg, fp8, routing, with_shared = case
    seed = 9000 + EDGE.index(case)
    rng = np.random.default_rng(seed)
    if routing == "zipf":
        import dataclasses
        cfg = dataclasses.replace(cfg, routing="zipf", target_maxvio=20.0)
    w = make_workload(cfg, seed=seed) if routing in (None, "zipf") else None
    hidden = make_workload(dataclasses_replace_uniform(cfg), seed=seed).hidden if w is None else w.hidden
    if routing == "all5":
        idx = np.full((cfg.S, cfg.K), 5, np.int32)
    elif routing == "bad":
        idx = rng.integers(0, cfg.E, (cfg.S, cfg.K)).astype(np.int32)
        hit = rng.random((cfg.S, cfg.K)) < 0.01
        idx[hit] = rng.choice([-1, cfg.E, cfg.E + 7, -100], int(hit.sum()))
    elif routing == "dup":
        idx = rng.integers(0, cfg.E, (cfg.S, cfg.K)).astype(np.int32)
    else:
        idx = w.topk_idx
    tw = rng.random((cfg.S, cfg.K)).astype(np.float32)
    tw /= tw.sum(axis=1, keepdims=True)
    shared = make_workload(dataclasses_replace_uniform(cfg), seed=seed + 1).hidden if with_shared else None
    ref = run_and_check(moe, cfg, idx, hidden, tw, shared=shared, fp8=fp8, seed=seed)
    if routing == "bad":
        assert ref.status[0] & oracle.FLAG_BAD_EXPERT
    if cfg.name == "multi-capacity-overflow":
        assert ref.status[0] & oracle.FLAG_CAPACITY


def dataclasses_replace_uniform(cfg):
    import dataclasses
    return dataclasses.replace(cfg, routing="uniform", K=min(cfg.K, cfg.E))


@pytest.mark.parametrize("E", [8, 256])   # single-workgroup and small-batch layouts
def test_empty_batch(moe, E):
    for pad_mode, pad_rows in ((PAD_NONE, 0), (PAD_MULTIPLE, 4), (PAD_CAPACITY, 3)):
        say(f"case empty: E={E} pad={pad_mode}/{pad_rows}")
        desc = moe.LayoutDesc(0, 2, E, 2, pad_mode, pad_rows)
        idx = torch.empty((0, 2), dtype=torch.int32, device=DEV)
        lay = moe.alloc_layout(desc, DEV)
        lay.status.fill_(-1)
        lay.src.fill_(7)
        moe.moe_layout(desc, idx, lay)
        torch.cuda.synchronize()
        compare_layout(lay, oracle.layout(np.zeros((0, 2), np.int32), E, 2, pad_mode, pad_rows), "empty")
        hid = torch.empty((0, 64), dtype=torch.bfloat16, device=DEV)
        moe.moe_dispatch(desc, lay, hid)
        y = torch.zeros((max(moe.moe_max_recv_rows(desc), 1), 64), dtype=torch.bfloat16, device=DEV)
        out = moe.moe_combine(desc, lay, y)
        assert out.shape == (0, 64)


def test_fp8_converter_sweep(moe):
    """Every finite bf16 value with |v| <= 448, in 128-channel blocks whose first
    element is +-448 (scale exactly 1, so the quotient is the value itself):
    the hardware E4M3 conversion against the oracle's encoder, bit for bit.
    This covers every E4M3 rounding midpoint (they are bf16 values), ties,
    subnormals, signed zeros and the saturation edge."""
    b = np.arange(0x8000, dtype=np.uint32)
    vals = (b << 16).view(np.float32)
    keep = b[np.abs(vals) <= 448.0].astype(np.uint16)
    allv = np.concatenate([keep, keep | np.uint16(0x8000)])
    per = 127
    nblk = -(-allv.size // per)
    H = 7168
    rows = -(-nblk // (H // 128))
    blocks = np.zeros((rows * (H // 128), 128), np.uint16)
    blocks[:, 0] = np.where(np.arange(blocks.shape[0]) % 2 == 0, 0x43E0, 0xC3E0)   # +448 / -448
    body = np.zeros(blocks.shape[0] * per, np.uint16)
    body[:allv.size] = allv
    blocks[:, 1:] = body.reshape(-1, per)
    hidden = blocks.reshape(rows, H)
    cfg = _case("fp8-sweep", rows, H, 1, 1, 1)
    idx = np.zeros((rows, 1), np.int32)
    tw = np.ones((rows, 1), np.float32)
    say(f"case fp8-sweep: {allv.size} bf16 values in {rows} rows")
    desc = moe.LayoutDesc(rows, 1, 1, 1)
    lay = moe.moe_layout(desc, torch.from_numpy(idx).to(DEV))
    recv, scales, _ = moe.moe_dispatch(desc, lay, dev_bf16(hidden, DEV), fp8=True)
    torch.cuda.synchronize()
    ref = oracle.layout(idx, 1, 1)
    rc, rs, _ = oracle.dispatch_fp8(hidden, ref.pos, rows)
    assert np.all(rs == 1.0)
    got = recv.cpu().numpy()
    bad = np.nonzero(got.reshape(-1) != rc.reshape(-1))[0]
    hv = hidden.reshape(-1)
    assert bad.size == 0, [(hex(int(hv[i])), int(got.reshape(-1)[i]), int(rc.reshape(-1)[i])) for i in bad[:8]]
    assert np.array_equal(scales.cpu().numpy(), rs)
    del cfg, tw


def test_combine_rounding_order_pins(moe):
    """Hand-worked cases where only an fp32 fma chain in ascending k gives the
    right bf16 bit (the same cases pin the oracle): 1+2^-8 then
    0x1.fc07f2p-25 * (1+2^-7) -> 0x3F81; 1+2^-8, 3*2^-26, 3*2^-26 -> 0x3F80;
    and one where only adding the shared output after the chain does."""
    H = 8
    one, one_p = 0x3F80, 0x3F81
    for ws, ys, want in (([1 + 2 ** -8, float.fromhex("0x1.fc07f2p-25")], [one, one_p], 0x3F81),
                         ([1 + 2 ** -8, 3 * 2 ** -26, 3 * 2 ** -26], [one, one, one], 0x3F80)):
        K = len(ws)
        say(f"case order-pin K={K}")
        desc = moe.LayoutDesc(1, K, K, 1)
        idx = torch.arange(K, dtype=torch.int32, device=DEV).reshape(1, K)
        lay = moe.moe_layout(desc, idx)
        y = np.repeat(np.array(ys, np.uint16)[:, None], H, axis=1)
        out = moe.moe_combine(desc, lay, dev_bf16(y, DEV), torch.tensor([ws], dtype=torch.float32, device=DEV))
        assert host_bits(out).tolist() == [[want] * H]
    # the shared output is added after the routed chain: 2^-8+3*2^-26 and
    # 3*2^-26 (y = 1.0) plus shared 1.0 -> 0x3F81 (shared first would give 0x3F80)
    say("case order-pin shared-last")
    desc = moe.LayoutDesc(1, 2, 2, 1)
    lay = moe.moe_layout(desc, torch.arange(2, dtype=torch.int32, device=DEV).reshape(1, 2))
    y = np.full((2, H), one, np.uint16)
    ws = torch.tensor([[2 ** -8 + 3 * 2 ** -26, 3 * 2 ** -26]], dtype=torch.float32, device=DEV)
    out = moe.moe_combine(desc, lay, dev_bf16(y, DEV), ws, shared_out=dev_bf16(np.full((1, H), one, np.uint16), DEV))
    assert host_bits(out).tolist() == [[0x3F81] * H]


def test_round_trip_on_gpu(moe):
    """combine(dispatch(x)) on the GPU alone, identity experts, weights summing
    to 1: x comes back bit for bit (a -0.0 input comes back as +0.0)."""
    cfg = CONFIGS["dsmoe16b"]
    w = make_workload(cfg)
    say("case round-trip dsmoe16b")
    desc = moe.LayoutDesc(cfg.S, cfg.K, cfg.E, cfg.R)
    lay = moe.moe_layout(desc, torch.from_numpy(w.topk_idx).to(DEV))
    tw = torch.from_numpy(w.topk_w).to(DEV)
    recv, _, _ = moe.moe_dispatch(desc, lay, dev_bf16(w.hidden, DEV), topk_w=tw)
    out = moe.moe_combine(desc, lay, recv, tw)
    want = np.where((w.hidden & 0x7FFF) == 0, 0, w.hidden)
    assert np.array_equal(host_bits(out), want)


def test_determinism_and_streams(moe):
    """Two runs, one on a side stream, give identical bits."""
    cfg = CONFIGS["prefill"]
    w = make_workload(cfg)
    say("case determinism prefill")
    desc = moe.LayoutDesc(cfg.S, cfg.K, cfg.E, cfg.R)
    idx = torch.from_numpy(w.topk_idx).to(DEV)
    hid = dev_bf16(w.hidden, DEV)
    torch.cuda.synchronize()
    outs = []
    side = torch.cuda.Stream()
    for stream in (None, side):
        with torch.cuda.stream(stream if stream is not None else torch.cuda.current_stream()):
            lay = moe.moe_layout(desc, idx, stream=stream)
            recv, sc, _ = moe.moe_dispatch(desc, lay, hid, fp8=True, stream=stream)
        torch.cuda.synchronize()
        outs.append((lay.pos.cpu().numpy(), lay.src.cpu().numpy(), recv.cpu().numpy(), sc.cpu().numpy()))
    for a, b in zip(*outs):
        assert np.array_equal(a, b)


def test_buffer_api(moe):
    """The static-shape Buffer (prepared calls) gives the same bits as the oracle."""
    for name in ("tiny", "decode"):
        cfg = CONFIGS[name]
        w = make_workload(cfg)
        say(f"case buffer-api {name}")
        buf = moe.Buffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=cfg.fp8, pad_mode=cfg.pad_mode,
                         pad_rows=cfg.pad_rows, device=DEV)
        idx = torch.from_numpy(w.topk_idx).to(DEV)
        tw = torch.from_numpy(w.topk_w).to(DEV)
        recv, recv_w, eoff, scales = buf.dispatch(dev_bf16(w.hidden, DEV), tw, idx)
        torch.cuda.synchronize()
        ref = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
        compare_layout(buf.layout, ref, "buffer layout")
        valid = ref.src >= 0
        if cfg.fp8:
            rc, rs, rw = oracle.dispatch_fp8(w.hidden, ref.pos, len(ref.src), w.topk_w)
            assert np.array_equal(recv.cpu().numpy()[valid], rc[valid])
            assert np.array_equal(scales.cpu().numpy()[valid], rs[valid])
            y = oracle.dequant_identity_expert(rc, rs)
        else:
            rb, rw = oracle.dispatch_bf16(w.hidden, ref.pos, len(ref.src), w.topk_w)
            assert np.array_equal(host_bits(recv)[valid], rb[valid])
            y = rb
        assert np.array_equal(recv_w.cpu().numpy()[valid], rw[valid])
        y = np.where(valid[:, None], y, np.uint16(POISON_BF16)).astype(np.uint16)
        out = buf.combine(dev_bf16(y, DEV), tw)
        torch.cuda.synchronize()
        assert_combine_matches(host_bits(out), oracle.combine(y, ref.pos, w.topk_w), "buffer combine")


@pytest.mark.parametrize("name", ["prefill", "skew"])
def test_bench_step(moe, name):
    """The exact sequence bench.py times (its Run: static Buffer, prepared
    layout, dispatch and combine calls without argument checks) at full size:
    every output against the oracle, combine over the bench's own expert
    outputs."""
    import bench
    cfg = CONFIGS[name]
    say(f"case bench-step {name}")
    run = bench.Run(moe, cfg, torch.device(DEV))
    run.buf.recv.zero_()
    run.step()
    torch.cuda.synchronize()
    w = run.w
    ref = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    compare_layout(run.buf.layout, ref, f"bench {name} layout")
    rows = len(ref.src)
    valid = ref.src >= 0
    if cfg.fp8:
        rc, rs, rw = oracle.dispatch_fp8(w.hidden, ref.pos, rows, w.topk_w)
        assert np.array_equal(run.buf.recv.cpu().numpy()[valid], rc[valid]), "fp8 codes"
        assert np.array_equal(run.buf.recv_scales.cpu().numpy()[valid].view(np.uint32),
                              rs[valid].view(np.uint32)), "fp8 scales"
    else:
        rb, rw = oracle.dispatch_bf16(w.hidden, ref.pos, rows, w.topk_w)
        assert np.array_equal(host_bits(run.buf.recv)[valid], rb[valid]), "bf16 rows"
    assert np.array_equal(run.buf.recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))
    y = host_bits(run.expert_out)
    assert_combine_matches(host_bits(run.buf.out), oracle.combine(y, ref.pos, w.topk_w, w.shared),
                           f"bench {name} combine")


@pytest.mark.parametrize("name", ["decode", "skew"])
def test_zero_padding(moe, name):
    """moe_zero_padding after dispatch: the whole receive buffer (and FP8
    scales), padding rows included, equals the oracle's dispatch followed by its
    zero padding, bit for bit."""
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    say(f"case zero-padding {name}")
    desc = moe.LayoutDesc(cfg.S, cfg.K, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    rows = moe.moe_max_recv_rows(desc)
    idx = torch.from_numpy(w.topk_idx).to(DEV)
    lay = moe.moe_layout(desc, idx)
    ref = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    pad = ref.src < 0
    assert pad.any()
    if cfg.fp8:
        recv = torch.full((rows, cfg.H), POISON_U8, dtype=torch.uint8, device=DEV)
        scales = torch.full((rows, cfg.H // 128), float("nan"), dtype=torch.float32, device=DEV)
        moe.moe_dispatch(desc, lay, dev_bf16(w.hidden, DEV), idx, fp8=True, recv=recv, recv_scales=scales)
        moe.moe_zero_padding(desc, lay, recv, scales)
        torch.cuda.synchronize()
        rc, rs, _ = oracle.dispatch_fp8(w.hidden, ref.pos, rows)
        want_c, want_s = oracle.zero_padding(ref.src, rc, rs)
        assert np.array_equal(recv.cpu().numpy(), want_c)
        assert np.array_equal(scales.cpu().numpy().view(np.uint32), want_s.view(np.uint32))
        # the same through Buffer's prepared call
        buf = moe.Buffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=True, pad_mode=cfg.pad_mode,
                         pad_rows=cfg.pad_rows, device=DEV)
        buf.recv.fill_(POISON_U8)
        buf.dispatch(dev_bf16(w.hidden, DEV), torch.from_numpy(w.topk_w).to(DEV), idx)
        buf.zero_padding_call()
        torch.cuda.synchronize()
        assert np.array_equal(buf.recv.cpu().numpy(), want_c)
    else:
        recv = torch.full((rows, cfg.H), POISON_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        moe.moe_dispatch(desc, lay, dev_bf16(w.hidden, DEV), idx, fp8=False, recv=recv)
        moe.moe_zero_padding(desc, lay, recv)
        torch.cuda.synchronize()
        rb, _ = oracle.dispatch_bf16(w.hidden, ref.pos, rows)
        want, _ = oracle.zero_padding(ref.src, rb)
        assert np.array_equal(host_bits(recv), want)


def test_ping_pong_buffer(moe):
    """Two decode calls back to back through PingPongBuffer: the first call's
    results are still exact after the second call ran."""
    cfg = CONFIGS["decode"]
    say("case ping-pong decode")
    pp = moe.PingPongBuffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=True, pad_mode=cfg.pad_mode,
                            pad_rows=cfg.pad_rows, device=DEV)
    calls = []
    for seed in (31, 32):
        w = make_workload(cfg, seed=seed)
        buf = pp.next()
        buf.dispatch(dev_bf16(w.hidden, DEV), torch.from_numpy(w.topk_w).to(DEV),
                     torch.from_numpy(w.topk_idx).to(DEV))
        calls.append((w, buf))
    assert calls[0][1] is not calls[1][1] and pp.next() is calls[0][1]
    torch.cuda.synchronize()
    for w, buf in calls:
        ref = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
        compare_layout(buf.layout, ref, "ping-pong layout")
        valid = ref.src >= 0
        rc, rs, rw = oracle.dispatch_fp8(w.hidden, ref.pos, len(ref.src), w.topk_w)
        assert np.array_equal(buf.recv.cpu().numpy()[valid], rc[valid])
        assert np.array_equal(buf.recv_scales.cpu().numpy()[valid].view(np.uint32), rs[valid].view(np.uint32))
        assert np.array_equal(buf.recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))


@pytest.mark.parametrize("form", ["three-calls", "fused"])
def test_graph_replay(moe, form):
    """Layout + dispatch + combine captured once in a HIP graph and replayed on
    three different batches, with eager work between the replays: every replay
    matches the eager result for its batch (no memset nodes are recorded: the
    layout kernels write every output they own).  Both forms of the decode
    call: three calls, and moe_layout_dispatch (one launch) + combine."""
    cfg = CONFIGS["decode"]
    say(f"case graph-replay decode {form}")
    buf = moe.Buffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=True, pad_mode=cfg.pad_mode,
                     pad_rows=cfg.pad_rows, device=DEV)
    idx = torch.empty((cfg.S, cfg.K), dtype=torch.int32, device=DEV)
    hid = torch.empty((cfg.S, cfg.H), dtype=torch.bfloat16, device=DEV)
    tw = torch.empty((cfg.S, cfg.K), dtype=torch.float32, device=DEV)
    y = torch.randn((buf.rows, cfg.H), device=DEV).to(torch.bfloat16)

    def load(seed):
        w = make_workload(cfg, seed=seed)
        idx.copy_(torch.from_numpy(w.topk_idx))
        hid.copy_(dev_bf16(w.hidden, DEV))
        tw.copy_(torch.from_numpy(w.topk_w))

    def step():
        if form == "fused":
            buf.layout_dispatch_call(hid, idx, tw, check=False)
        else:
            buf.layout_call(idx, check=False)
            buf.dispatch_call(hid, idx, tw, check=False)
        buf.combine_call(y, tw, check=False)

    def snapshot():
        return [t.clone() for t in (buf.layout.pos, buf.layout.src, buf.layout.expert_offset, buf.recv,
                                    buf.recv_scales, buf.recv_w, buf.out)]

    load(1)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    def reset():   # rows nobody writes (padding) must start equal for both runs
        for t in (buf.recv, buf.recv_scales, buf.recv_w, buf.out):
            t.zero_()
        buf.layout.pos.fill_(-7)

    for seed in (11, 12, 13):
        load(seed)
        reset()
        step()                          # eager reference for this batch
        torch.cuda.synchronize()
        want = snapshot()
        reset()
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = snapshot()
        for a, b in zip(got, want):
            assert torch.equal(a, b)


@pytest.mark.parametrize("S", [2000, 5000], ids=["one-launch-N16000", "two-step-N40000"])
def test_buffer_balanced(moe, S):
    """Buffer with balance_slots: its prepared calls (balanced layout, FP8
    dispatch, combine) against the oracle, every output bit for bit."""
    K, E, R, B, H = 8, 64, 8, 4, 256
    cfg = _case("buffer-balanced", S, H, E, K, R, routing="zipf")
    w = make_workload(cfg)
    say(f"case buffer-balanced S={S}")
    buf = moe.Buffer(S, H, K, E, R, fp8=True, device=DEV, balance_slots=B)
    idx = torch.from_numpy(w.topk_idx).to(DEV)
    tw = torch.from_numpy(w.topk_w).to(DEV)
    recv, recv_w, eoff, scales = buf.dispatch(dev_bf16(w.hidden, DEV), tw, idx)
    torch.cuda.synchronize()
    ref = oracle.layout_balanced(w.topk_idx, E, R, B)
    for k in ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status"):
        want = getattr(ref, k)
        assert np.array_equal(getattr(buf.layout, k).cpu().numpy().reshape(want.shape), want), k
    assert np.array_equal(buf.balance.seg_offset.cpu().numpy(), ref.seg_offset)
    assert np.array_equal(buf.balance.slot_expert.cpu().numpy()[:R * B], ref.slot_expert)
    assert int((ref.slot_expert >= 0).sum()) > 0, "the batch should need replicas"
    valid = ref.src >= 0
    rc, rs, rw = oracle.dispatch_fp8(w.hidden, ref.pos, len(ref.src), w.topk_w)
    assert np.array_equal(recv.cpu().numpy()[valid], rc[valid])
    assert np.array_equal(scales.cpu().numpy()[valid].view(np.uint32), rs[valid].view(np.uint32))
    assert np.array_equal(recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))
    y = random_expert_out_bits(w.seed, len(ref.src), H, row_mask=valid, poison=POISON_BF16)
    out = buf.combine(dev_bf16(y, DEV), tw)
    torch.cuda.synchronize()
    assert_combine_matches(host_bits(out), oracle.combine(y, ref.pos, w.topk_w), "buffer balanced combine")


@pytest.mark.parametrize("S", [2000, 5000], ids=["one-launch-N16000", "two-step-N40000"])
def test_graph_replay_balanced(moe, S):
    """The balanced layout captured in a HIP graph and replayed on three
    batches: every replay equals the eager call for that batch."""
    K, E, R, B = 8, 64, 8, 4
    say(f"case graph-replay balanced S={S}")
    desc = moe.LayoutDesc(S, K, E, R)
    lay = moe.alloc_layout(desc, DEV)
    bal = moe.alloc_balance(desc, B, DEV)
    idx = torch.empty((S, K), dtype=torch.int32, device=DEV)
    cfg = _case("graph-bal", S, 8, E, K, R, routing="zipf")

    def step():
        moe.moe_layout_balanced(desc, B, idx, lay, bal)

    def snapshot():
        return [t.clone() for t in (lay.pos, lay.src, lay.expert_offset, lay.tokens_per_rank, lay.status,
                                    bal.seg_offset, bal.slot_expert)]

    idx.copy_(torch.from_numpy(make_workload(cfg, seed=1, with_hidden=False).topk_idx))
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        step()
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step()
    torch.cuda.synchronize()
    for seed in (21, 22, 23):
        idx.copy_(torch.from_numpy(make_workload(cfg, seed=seed, with_hidden=False).topk_idx))
        for t in (lay.pos, lay.src):
            t.fill_(-7)
        step()
        torch.cuda.synchronize()
        want = snapshot()
        for t in (lay.pos, lay.src):
            t.fill_(-7)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for a, b in zip(snapshot(), want):
            assert torch.equal(a, b)


FUSED = [
    # name, S, H, E, K, R, pad_mode, pad_rows, fp8, routing
    ("decode", 128, 7168, 256, 8, 8, PAD_CAPACITY, 128, True, "uniform"),
    ("tiny-bf16", 256, 512, 16, 2, 4, PAD_NONE, 0, False, "uniform"),
    ("max-fused-N4096-E1024-K16", 256, 256, 1024, 16, 8, PAD_MULTIPLE, 5, True, "uniform"),
    ("fallback-N4104", 513, 128, 64, 8, 8, PAD_NONE, 0, True, "uniform"),
    ("fallback-multi-N20000", 2500, 64, 32, 8, 4, PAD_MULTIPLE, 16, False, "uniform"),
    ("capacity-overflow", 300, 1024, 16, 8, 4, PAD_CAPACITY, 100, True, "uniform"),
    ("bad-ids", 200, 136, 32, 4, 2, PAD_NONE, 0, False, "bad"),
    ("duplicates", 100, 8, 4, 6, 2, PAD_MULTIPLE, 3, False, "dup"),
    ("one-token", 1, 128, 1, 1, 1, PAD_NONE, 0, True, "uniform"),
    # the one-launch form's token limit (S <= 512) at S*K <= 4096
    ("fused-S512-N4096", 512, 1024, 256, 8, 8, PAD_CAPACITY, 20, True, "uniform"),
    ("fallback-S513-N3591", 513, 1024, 128, 7, 8, PAD_MULTIPLE, 4, False, "uniform"),
    # rows wider than one workgroup's slice (several chunks per token, ragged last one)
    ("wide-fp8-H16512", 48, 16512, 32, 4, 4, PAD_CAPACITY, 12, True, "uniform"),
    ("wide-bf16-H8200", 64, 8200, 16, 2, 2, PAD_NONE, 0, False, "uniform"),
]


def _random_fused(n=20, seed=5151):
    """Seeded random decode-sized shapes for moe_layout_dispatch (most within
    S*K <= 4096, some just past it; the one-launch form also needs S <= 512)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        fp8 = bool(rng.integers(0, 2))
        H = int(rng.integers(1, 9)) * 128 if fp8 else int(rng.integers(1, 129)) * 8
        R = int(rng.choice([1, 2, 4, 8]))
        E = R * int(rng.integers(1, 1024 // R + 1))
        routing = str(rng.choice(["uniform", "uniform", "dup", "bad"]))
        K = int(rng.integers(1, min(16, E) + 1)) if routing == "uniform" else int(rng.integers(1, 17))
        N = int(rng.integers(1, 4097)) if i % 5 else int(rng.integers(4097, 6000))
        S = max(1, N // K)
        pad = int(rng.integers(0, 3))
        pad_rows = {PAD_NONE: 0, PAD_MULTIPLE: int(rng.integers(1, 130)),
                    PAD_CAPACITY: int(max(1, S * K // E * rng.uniform(0.5, 2.0)))}[pad]
        out.append((f"rand-fused{i}", S, H, E, K, R, pad, pad_rows, fp8, routing))
    return out


FUSED += _random_fused()


@pytest.mark.parametrize("case", FUSED, ids=[c[0] for c in FUSED])
def test_layout_dispatch(moe, case):
    """moe_layout_dispatch (one launch for S*K <= 4096 and S <= 512, two
    otherwise) against the oracle's layout + dispatch, every output bit for
    bit."""
    name, S, H, E, K, R, pad_mode, pad_rows, fp8, routing = case
    seed = 7000 + FUSED.index(case)
    rng = np.random.default_rng(seed)
    cfg = _case(name, S, H, E, K, R, pad_mode, pad_rows)
    hidden = make_workload(dataclasses_replace_uniform(cfg), seed=seed).hidden
    if routing == "uniform":
        idx = make_workload(cfg, seed=seed).topk_idx
    else:
        idx = rng.integers(0, E, (S, K)).astype(np.int32)
        if routing == "bad":
            hit = rng.random((S, K)) < 0.02
            idx[hit] = rng.choice([-1, E, 1 << 30], int(hit.sum()))
    tw = rng.random((S, K)).astype(np.float32)
    say(f"case layout-dispatch {name}: S={S} H={H} E={E} K={K} fp8={fp8}")
    desc = moe.LayoutDesc(S, K, E, R, pad_mode, pad_rows)
    rows = moe.moe_max_recv_rows(desc)
    ref = oracle.layout(idx, E, R, pad_mode, pad_rows)
    valid = ref.src >= 0
    if fp8:
        recv = torch.full((rows, H), POISON_U8, dtype=torch.uint8, device=DEV)
        scales = torch.full((rows, H // 128), float("nan"), dtype=torch.float32, device=DEV)
    else:
        recv = torch.full((rows, H), POISON_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        scales = None
    recv_w = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    lay, _, _, _ = moe.moe_layout_dispatch(desc, torch.from_numpy(idx).to(DEV), dev_bf16(hidden, DEV),
                                           torch.from_numpy(tw).to(DEV), fp8=fp8, recv=recv,
                                           recv_scales=scales, recv_w=recv_w)
    torch.cuda.synchronize()
    compare_layout(lay, ref, f"{name} layout")
    if fp8:
        rc, rs, rw = oracle.dispatch_fp8(hidden, ref.pos, rows, tw)
        got = recv.cpu().numpy()
        assert np.array_equal(got[valid], rc[valid])
        assert np.array_equal(scales.cpu().numpy()[valid].view(np.uint32), rs[valid].view(np.uint32))
        assert np.all(got[~valid] == POISON_U8)
    else:
        rb, rw = oracle.dispatch_bf16(hidden, ref.pos, rows, tw)
        got = host_bits(recv)
        assert np.array_equal(got[valid], rb[valid])
        assert np.all(got[~valid] == POISON_BF16)
    assert np.array_equal(recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))
    assert np.all(np.isnan(recv_w.cpu().numpy()[~valid]))


def test_cu_limited_stream(moe):
    """Layout, FP8 dispatch and combine on CU-limited streams (the first 16 and
    32 CUs, and the upper half of the chip as a placed range), each checked
    against the oracle: layout and FP8 codes and scales bit for bit, combine of
    seeded random expert outputs within one bf16 ulp."""
    cfg = CONFIGS["prefill"]
    w = make_workload(cfg)
    say("case cu-limited stream prefill: oracle")
    ref = oracle.layout(w.topk_idx, cfg.E, cfg.R)
    rows = len(ref.src)
    valid = ref.src >= 0
    rc, rs, rw = oracle.dispatch_fp8(w.hidden, ref.pos, rows, w.topk_w)
    y = random_expert_out_bits(w.seed, rows, cfg.H, row_mask=valid, poison=POISON_BF16)
    out_ref = oracle.combine(y, ref.pos, w.topk_w)
    buf = moe.Buffer(cfg.S, cfg.H, cfg.K, cfg.E, cfg.R, fp8=True, device=DEV)
    assert buf.rows == rows
    idx = torch.from_numpy(w.topk_idx).to(DEV)
    hid = dev_bf16(w.hidden, DEV)
    tw = torch.from_numpy(w.topk_w).to(DEV)
    y_d = dev_bf16(y, DEV)
    n_cu = torch.cuda.get_device_properties(0).multi_processor_count
    for first, count in ((0, 16), (0, 32), (n_cu // 2, n_cu // 2)):
        say(f"case cu-limited stream prefill: CUs [{first}, {first + count})")
        for lt in (buf.layout.pos, buf.layout.src, buf.layout.tokens_per_expert, buf.layout.expert_offset):
            lt.fill_(-7)
        buf.recv.fill_(POISON_U8)
        buf.recv_scales.fill_(float("nan"))
        buf.recv_w.fill_(float("nan"))
        buf.out.view(torch.int16).fill_(POISON_BF16)
        torch.cuda.synchronize()
        with moe.CULimitedStream(count, DEV, first_cu=first) as cs:
            with torch.cuda.stream(cs.stream):
                buf.layout_call(idx)
                buf.dispatch_call(hid, idx, tw)
                buf.combine_call(y_d, tw)
            torch.cuda.synchronize()
        compare_layout(buf.layout, ref, f"layout on {count} CUs")
        got_c, got_s = buf.recv.cpu().numpy(), buf.recv_scales.cpu().numpy()
        assert np.array_equal(got_c[valid], rc[valid]), f"fp8 codes on {count} CUs"
        assert np.array_equal(got_s[valid].view(np.uint32), rs[valid].view(np.uint32)), f"fp8 scales on {count} CUs"
        assert np.array_equal(buf.recv_w.cpu().numpy()[valid].view(np.uint32), rw[valid].view(np.uint32))
        assert_combine_matches(host_bits(buf.out), out_ref, f"combine on {count} CUs")
    # ranges the XCD rule refuses
    handle = ctypes.c_void_p()
    lib = moe.lib()
    assert lib.moe_stream_create_cu_range(4, 32, ctypes.byref(handle)) == moe.MOE_ERR_SHAPE
    assert lib.moe_stream_create_cu_range(n_cu - 8, 16, ctypes.byref(handle)) == moe.MOE_ERR_SHAPE


BAL = [
    # name, S, K, E, R, B, routing
    ("skew-B16", 4096, 8, 256, 8, 16, "skew"),
    ("skew-B8-unbalanced", 4096, 8, 256, 8, 8, "skew"),
    ("random-small", 300, 4, 32, 4, 3, "pow"),
    ("random-bad-ids", 1000, 6, 64, 8, 4, "bad"),
    ("one-rank", 500, 2, 16, 1, 4, "pow"),
    ("no-slots", 700, 3, 24, 4, 0, "pow"),
    ("E1024-R8-B64", 2000, 8, 1024, 8, 64, "pow"),
    ("big-N100000-E96-R6", 12500, 8, 96, 6, 8, "pow"),
    ("big-bad-ids-N40000", 5000, 8, 64, 8, 4, "bad"),     # two-step path with invalid ids
    ("empty", 0, 4, 16, 4, 2, "pow"),
]


def _random_bal(n=16, seed=6161):
    """Seeded random balanced-layout shapes, both forms (one launch up to 32K
    entries, two steps above)."""
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        R = int(rng.choice([1, 2, 3, 4, 6, 8, 16]))
        E = R * int(rng.integers(1, 1024 // R + 1))
        K = int(rng.integers(1, 17))
        N = int(rng.integers(1, 32769)) if i % 4 else int(rng.integers(32769, 70000))
        S = max(1, N // K)
        B = int(rng.integers(0, min(64, 512 // R) + 1))
        out.append((f"rand-bal{i}", S, K, E, R, B, str(rng.choice(["pow", "pow", "bad"]))))
    return out


BAL += _random_bal()


@pytest.mark.parametrize("case", BAL, ids=[c[0] for c in BAL])
def test_layout_balanced(moe, case):
    """Balanced layout (redundant-expert slots) against the oracle, every output
    bit for bit; then bf16 dispatch and combine through the balanced maps."""
    name, S, K, E, R, B, routing = case
    seed = 8000 + BAL.index(case)
    rng = np.random.default_rng(seed)
    if routing == "skew":
        w = make_workload(CONFIGS["skew"])
        idx, hidden, tw = w.topk_idx, w.hidden, w.topk_w
        H = 1024
        hidden = np.ascontiguousarray(hidden[:, :H])
    else:
        H = 64
        p = rng.random(E) ** 3
        idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
        if routing == "bad" and idx.size:
            idx.reshape(-1)[rng.integers(0, idx.size, 20)] = -1
        hidden = make_workload(_case(name, max(S, 1), H, E, 1, 1), seed=seed).hidden[:S]
        tw = rng.random((S, K)).astype(np.float32)
    say(f"case balanced {name}: S={S} K={K} E={E} R={R} B={B}")
    desc = moe.LayoutDesc(S, K, E, R)
    lay, bal = moe.moe_layout_balanced(desc, B, torch.from_numpy(np.ascontiguousarray(idx)).to(DEV))
    torch.cuda.synchronize()
    ref = oracle.layout_balanced(idx, E, R, B)
    for k in ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status"):
        want = getattr(ref, k)
        got = getattr(lay, k).cpu().numpy().reshape(want.shape)
        assert np.array_equal(got, want), k
    assert np.array_equal(bal.seg_offset.cpu().numpy(), ref.seg_offset)
    if B > 0:
        assert np.array_equal(bal.slot_expert.cpu().numpy()[:R * B], ref.slot_expert)
    if routing == "skew":
        assert (int(ref.status[0]) & oracle.FLAG_UNBALANCED) == (0 if B == 16 else oracle.FLAG_UNBALANCED)
    if S == 0:
        return
    # dispatch and combine take the balanced maps unchanged
    rows = moe.moe_max_recv_rows(desc)
    valid = ref.src >= 0
    recv = torch.full((rows, H), POISON_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    tw_d = torch.from_numpy(np.ascontiguousarray(tw)).to(DEV)
    moe.moe_dispatch(desc, lay, dev_bf16(hidden, DEV), topk_w=tw_d, recv=recv)
    torch.cuda.synchronize()
    rb, _ = oracle.dispatch_bf16(hidden, ref.pos, rows, tw)
    assert np.array_equal(host_bits(recv)[valid], rb[valid])
    y = random_expert_out_bits(seed, rows, H, row_mask=valid, poison=POISON_BF16)
    out = moe.moe_combine(desc, lay, dev_bf16(y, DEV), tw_d)
    torch.cuda.synchronize()
    assert_combine_matches(host_bits(out), oracle.combine(y, ref.pos, tw), "balanced combine")


# name, S, K, E, R, pad mode, pad rows: entry counts S*K that are not multiples of
# 4, in the single-workgroup, small-batch, one-launch and two-launch layouts
IDX_OFFSET = [
    ("single-N1999", 1999, 1, 32, 4, PAD_NONE, 0),
    ("small-N4093", 4093, 1, 256, 8, PAD_CAPACITY, 24),
    ("onepass-N9999", 3333, 3, 256, 8, PAD_NONE, 0),
    ("onepass-N30002", 15001, 2, 64, 8, PAD_MULTIPLE, 16),
    ("onepass-N32767", 32767, 1, 128, 4, PAD_NONE, 0),
    ("multi-N40001", 40001, 1, 96, 6, PAD_NONE, 0),
    # the count's 4- and 2-copy counters (E in (256, 512] and (512, 1024])
    ("onepass-N20001-E264", 20001, 1, 264, 8, PAD_CAPACITY, 70),
    ("onepass-N9003-E1000", 3001, 3, 1000, 8, PAD_MULTIPLE, 2),
]


@pytest.mark.parametrize("offset", [0, 1], ids=["aligned", "idx-off-by-4-bytes"])
@pytest.mark.parametrize("case", IDX_OFFSET, ids=[c[0] for c in IDX_OFFSET])
def test_layout_idx_alignment(moe, case, offset):
    """topk_idx carries no alignment requirement: the layouts read it four
    entries at a time only when it is 16-byte aligned.  Both forms, with a
    ragged last group of four, against the oracle (plain and balanced)."""
    name, S, K, E, R, pad_mode, pad_rows = case
    seed = 7100 + IDX_OFFSET.index(case)
    rng = np.random.default_rng(seed)
    p = rng.random(E) ** 2
    idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
    idx.reshape(-1)[rng.integers(0, idx.size, 5)] = E + 3   # a few invalid ids
    say(f"case idx alignment {name} offset={offset}: S={S} K={K} E={E} R={R} pad={pad_mode}/{pad_rows}")
    store = torch.zeros(S * K + 4, dtype=torch.int32, device=DEV)
    view = store[offset:offset + S * K].view(S, K)
    view.copy_(torch.from_numpy(idx))
    assert (view.data_ptr() % 16 == 0) == (offset == 0)
    desc = moe.LayoutDesc(S, K, E, R, pad_mode, pad_rows)
    lay = moe.moe_layout(desc, view)
    torch.cuda.synchronize()
    compare_layout(lay, oracle.layout(idx, E, R, pad_mode, pad_rows), f"{name} layout")
    lay_b, bal = moe.moe_layout_balanced(moe.LayoutDesc(S, K, E, R), 4, view)
    torch.cuda.synchronize()
    ref = oracle.layout_balanced(idx, E, R, 4)
    for k in ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status"):
        want = getattr(ref, k)
        assert np.array_equal(getattr(lay_b, k).cpu().numpy().reshape(want.shape), want), f"balanced {k}"
    assert np.array_equal(bal.seg_offset.cpu().numpy(), ref.seg_offset)


def test_layout_random_sweep(moe):
    """2,000 seeded random layouts, plain and balanced, every output against the
    oracle: all layout variants (small, single, one-launch, two-launch), every
    pad mode, skewed and uniform routing, invalid ids, and topk_idx at every
    4-byte offset inside a 16-byte line."""
    rng = np.random.default_rng(20261203)
    for n in range(2000):
        R = int(rng.choice([1, 2, 4, 8, 16]))
        E = R * int(rng.integers(1, 1024 // R + 1))
        K = int(rng.integers(1, 17))
        N = int(rng.choice([rng.integers(1, 4097), rng.integers(4097, 32769), rng.integers(32769, 70000)]))
        S = max(1, N // K)
        pad_mode = int(rng.integers(0, 3))
        pad_rows = 0 if pad_mode == PAD_NONE else int(rng.integers(1, 200))
        p = rng.random(E) ** float(rng.choice([0.0, 1.0, 4.0]))
        idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
        if rng.random() < 0.3:
            idx.reshape(-1)[rng.integers(0, idx.size, 7)] = int(rng.choice([-1, E, E + 5]))
        offset = int(rng.integers(0, 4))
        B = int(rng.integers(0, min(64, 512 // R) + 1))
        case = f"sweep {n}: S={S} K={K} E={E} R={R} pad={pad_mode}/{pad_rows} offset={offset} B={B}"
        store = torch.zeros(S * K + 4, dtype=torch.int32, device=DEV)
        view = store[offset:offset + S * K].view(S, K)
        view.copy_(torch.from_numpy(idx))
        lay = moe.moe_layout(moe.LayoutDesc(S, K, E, R, pad_mode, pad_rows), view)
        torch.cuda.synchronize()
        compare_layout(lay, oracle.layout(idx, E, R, pad_mode, pad_rows), case)
        lay_b, _ = moe.moe_layout_balanced(moe.LayoutDesc(S, K, E, R), B, view)
        torch.cuda.synchronize()
        ref = oracle.layout_balanced(idx, E, R, B)
        for k in ("tokens_per_expert", "tokens_per_rank", "expert_offset", "rank_offset", "pos", "src", "status"):
            want = getattr(ref, k)
            assert np.array_equal(getattr(lay_b, k).cpu().numpy().reshape(want.shape), want), f"{case}: balanced {k}"


BEYOND_4GIB = [
    # bf16 rows of 14 KiB with padding: an 8.0 GB receive buffer (its last row
    # at byte 7.98e9), also read back by combine as the expert outputs
    (WorkloadConfig("beyond4g-bf16", S=65536, H=7168, E=256, K=8, R=8, routing="uniform",
                    pad_mode=PAD_MULTIPLE, pad_rows=128), False),
    # FP8 rows of 4,224 bytes: a 4.43 GB receive buffer, 1,048,576 entries
    # (the two-launch layout with its largest tiles)
    (WorkloadConfig("beyond4g-fp8", S=131072, H=4224, E=64, K=8, R=8, routing="uniform"), True),
]


@pytest.mark.parametrize("case", BEYOND_4GIB, ids=[c[0].name for c in BEYOND_4GIB])
def test_beyond_4gib(moe, case):
    """Receive buffers larger than 4 GiB: the whole layout bit-exact against
    the oracle, and sampled tokens -- random ones, the owners of the highest
    rows and of the rows around the 4 GiB byte boundary -- dispatched (and for
    bf16 combined from the receive buffer) exactly as the oracle computes them
    for those tokens alone.  Padding rows near the end must stay untouched."""
    from workloads import softmax_weights, stamped_rows_bf16_bits, uniform_distinct_routing
    cfg, fp8 = case
    S, H, E, K, R = cfg.S, cfg.H, cfg.E, cfg.K, cfg.R
    say(f"case {cfg.name}: S={S} H={H} E={E} K={K} fp8={fp8}")
    rng = np.random.default_rng(77)
    idx = uniform_distinct_routing(rng, S, E, K)
    w = softmax_weights(rng.standard_normal((S, K), dtype=np.float32))
    hidden = stamped_rows_bf16_bits(78, S, H)
    desc = moe.LayoutDesc(S, K, E, R, cfg.pad_mode, cfg.pad_rows)
    rows = moe.moe_max_recv_rows(desc)
    row_bytes = H if fp8 else 2 * H
    assert rows * row_bytes > (1 << 32)
    ref = oracle.layout(idx, E, R, cfg.pad_mode, cfg.pad_rows)
    assert rows == len(ref.src)

    idx_d = torch.from_numpy(idx).to(DEV)
    w_d = torch.from_numpy(w).to(DEV)
    hid_d = dev_bf16(hidden, DEV)
    lay = moe.moe_layout(desc, idx_d)
    torch.cuda.synchronize()
    compare_layout(lay, ref, f"{cfg.name} layout")
    say("  layout ok")

    if fp8:
        recv = torch.full((rows, H), POISON_U8, dtype=torch.uint8, device=DEV)
        scales = torch.full((rows, H // 128), float("nan"), dtype=torch.float32, device=DEV)
    else:
        recv = torch.full((rows, H), POISON_BF16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
        scales = None
    recv_w = torch.full((rows,), float("nan"), dtype=torch.float32, device=DEV)
    moe.moe_dispatch(desc, lay, hid_d, idx_d, w_d, fp8=fp8, recv=recv, recv_scales=scales, recv_w=recv_w)
    torch.cuda.synchronize()

    flat = ref.pos.reshape(-1)
    by_row = np.argsort(flat)
    boundary = (1 << 32) // row_bytes           # the row that straddles byte 2**32
    near = np.nonzero(np.abs(flat.astype(np.int64) - boundary) <= 2)[0]
    tokens = np.unique(np.concatenate([rng.choice(S, 384, replace=False), by_row[-64:] // K, near // K,
                                       [0, S - 1]]))
    assert int(flat[by_row[-1]]) * row_bytes > (1 << 32) and near.size > 0
    n = tokens.size
    pos_sub = np.arange(n * K, dtype=np.int32).reshape(n, K)
    sel = ref.pos[tokens].reshape(-1)
    recv_host = recv.view(torch.uint8) if fp8 else recv.view(torch.int16)
    got = np.stack([recv_host[int(r)].cpu().numpy() for r in sel])
    got_w = recv_w.cpu().numpy()[sel]
    if fp8:
        want, want_s, want_w = oracle.dispatch_fp8(hidden[tokens], pos_sub, n * K, w[tokens])
        got_s = np.stack([scales[int(r)].cpu().numpy() for r in sel])
        assert np.array_equal(got, want), "fp8 codes differ"
        assert np.array_equal(got_s.view(np.uint32), want_s.view(np.uint32)), "fp8 scales differ"
    else:
        want, want_w = oracle.dispatch_bf16(hidden[tokens], pos_sub, n * K, w[tokens])
        assert np.array_equal(got.view(np.uint16), want), "bf16 rows differ"
    assert np.array_equal(got_w.view(np.uint32), want_w.view(np.uint32)), "recv_w differs"
    pad_rows = np.nonzero(ref.src < 0)[0][-64:]
    for r in pad_rows:
        row = recv_host[int(r)].cpu().numpy()
        assert np.all(row.view(np.uint8 if fp8 else np.uint16) == (POISON_U8 if fp8 else POISON_BF16)), r
    say(f"  dispatch ok on {n} sampled tokens ({n * K} rows, last row {int(flat[by_row[-1]])}), "
        f"{pad_rows.size} padding rows untouched")

    if not fp8:
        out = moe.moe_combine(desc, lay, recv, w_d)
        torch.cuda.synchronize()
        got_o = host_bits(out[torch.from_numpy(tokens).to(DEV)])
        assert_combine_matches(got_o, oracle.combine(want, pos_sub, w[tokens]), "combine beyond 4 GiB")
        say("  combine ok")
        del out
    del recv, scales, recv_w, hid_d, lay
    torch.cuda.empty_cache()
