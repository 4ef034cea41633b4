"""The pattern-ceiling kernels (libmoe_ceilings.so) move the bytes they claim:
small buffers, every output byte checked against numpy.  These kernels only
time HBM patterns for the benchmark; the check makes sure a ceiling is
measured on the intended traffic."""
from __future__ import annotations

import numpy as np
import pytest
import torch

pytestmark = pytest.mark.gpu
DEV = "cuda:0"


@pytest.fixture(scope="module")
def pat():
    assert torch.cuda.is_available(), "GPU tests need a GPU"
    import bench
    return bench.Patterns(torch.device(DEV))


def _u32(t: torch.Tensor) -> np.ndarray:
    return t.cpu().numpy().view(np.uint32)


@pytest.mark.parametrize("v,w", [(1, 1), (4, 4), (16, 2)])
def test_read_write(pat, v, w):
    print(f"case ceilings read/write V={v} W={w}", flush=True)
    nbytes = 64 << 10
    buf = torch.ones(nbytes // 4, dtype=torch.float32, device=DEV)
    for kind in ("plain", "nt"):
        pat.read(buf, v, w, kind)()
    torch.cuda.synchronize()
    assert np.all(pat.sink.cpu().numpy() == 0)          # the data never matches the sink's key
    nvec = nbytes // 16
    g = np.arange(nvec)
    wave = g // (v * 64)
    lane = g % 64
    tid = (wave % w) * 64 + lane
    want = np.stack([wave, tid, np.full(nvec, 0x5EEDF00D), np.zeros(nvec)], axis=1).astype(np.uint32)
    for kind in ("plain", "nt", "sc1"):
        out = torch.zeros(nbytes // 4, dtype=torch.int32, device=DEV)
        pat.write(out, v, w, kind)()
        torch.cuda.synchronize()
        assert np.array_equal(_u32(out).reshape(nvec, 4), want), kind


@pytest.mark.parametrize("fp8,waves", [(False, 1), (True, 1), (False, 2), (True, 4)])
def test_scatter(pat, fp8, waves):
    print(f"case ceilings scatter fp8={fp8} waves={waves}", flush=True)
    S, K, out_rb = 6, 4, 4096
    in_rb = 2 * out_rb if fp8 else out_rb
    rng = np.random.default_rng(3)
    src = rng.integers(0, 2 ** 32, (S, in_rb // 4), dtype=np.uint64).astype(np.uint32)
    nrows = S * K + 5
    rows = rng.permutation(nrows)[:S * K].astype(np.int32).reshape(S, K)
    rows[2, 1] = -1
    src_d = torch.from_numpy(src.view(np.int32)).to(DEV)
    dst = torch.full((nrows, out_rb // 4), -1, dtype=torch.int32, device=DEV)
    sc = torch.full((nrows, out_rb // 128), -1, dtype=torch.int32, device=DEV) if fp8 else None
    pat.scatter(src_d.view(torch.uint8), torch.from_numpy(rows).to(DEV), dst.view(torch.uint8),
                sc.view(torch.float32) if fp8 else None, waves)()
    torch.cuda.synchronize()
    got = _u32(dst)
    vec = src.reshape(S, -1, 2, 4)
    x = (vec[:, :, 0] ^ vec[:, :, 1]) if fp8 else src.reshape(S, -1, 4)
    written = np.zeros(nrows, bool)
    for t in range(S):
        for k in range(K):
            r = rows[t, k]
            if r < 0:
                continue
            written[r] = True
            assert np.array_equal(got[r].reshape(-1, 4), x[t]), (t, k)
            if fp8:
                s = _u32(sc)[r]
                assert np.array_equal(s, x[t][::8, 0] & 0x3F7FFFFF), (t, k)
    assert np.all(got[~written] == 0xFFFFFFFF)


@pytest.mark.parametrize("fp8", [False, True])
def test_scatter_rows_matches_scatter(pat, fp8):
    """Row order through LDS writes the same bytes as the chunked scatter."""
    print(f"case ceilings scatter rows fp8={fp8}", flush=True)
    S, K, out_rb = 5, 8, 3072
    in_rb = 2 * out_rb if fp8 else out_rb
    rng = np.random.default_rng(6)
    src = rng.integers(0, 2 ** 32, (S, in_rb // 4), dtype=np.uint64).astype(np.uint32)
    nrows = S * K + 3
    rows = rng.permutation(nrows)[:S * K].astype(np.int32).reshape(S, K)
    rows[1, 5] = -1
    src_d = torch.from_numpy(src.view(np.int32)).to(DEV).view(torch.uint8)
    rows_d = torch.from_numpy(rows).to(DEV)
    outs = []
    for form in ("chunks", "rows"):
        dst = torch.full((nrows, out_rb // 4), -1, dtype=torch.int32, device=DEV)
        sc = torch.full((nrows, out_rb // 128), -1, dtype=torch.int32, device=DEV) if fp8 else None
        scf = sc.view(torch.float32) if fp8 else None
        if form == "chunks":
            pat.scatter(src_d, rows_d, dst.view(torch.uint8), scf)()
        else:
            pat.scatter_rows(src_d, rows_d, dst.view(torch.uint8), scf)()
        torch.cuda.synchronize()
        outs.append((_u32(dst), None if sc is None else _u32(sc)))
    assert np.array_equal(outs[0][0], outs[1][0])
    if fp8:
        assert np.array_equal(outs[0][1], outs[1][1])
    assert np.any(outs[0][0] != 0xFFFFFFFF)


@pytest.mark.parametrize("v", [1, 2])
def test_gather(pat, v):
    print(f"case ceilings gather V={v}", flush=True)
    S, K, rb = 5, 6, 4096
    rng = np.random.default_rng(4)
    nrows = 40
    y = rng.integers(0, 2 ** 32, (nrows, rb // 4), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(0, nrows, (S, K)).astype(np.int32)
    rows[1, 3] = -1
    y_d = torch.from_numpy(y.view(np.int32)).to(DEV)
    want = np.zeros((S, rb // 4), np.uint32)
    for t in range(S):
        for k in range(K):
            if rows[t, k] >= 0:
                want[t] ^= y[rows[t, k]]
    for kind in ("plain", "nt", "sc1"):
        out = torch.full((S, rb // 4), -1, dtype=torch.int32, device=DEV)
        pat.gather(y_d.view(torch.uint8), torch.from_numpy(rows).to(DEV), out.view(torch.uint8), v, kind)()
        torch.cuda.synchronize()
        assert np.array_equal(_u32(out), want), kind


@pytest.mark.parametrize("groups,waves", [(1, 1), (3, 2), (2, 4), (64, 4)])
def test_gather_persistent(pat, groups, waves):
    """Same bytes as the gather pattern, whatever the number of persistent
    waves (fewer waves than units, more waves than units)."""
    print(f"case ceilings gather persistent groups={groups} waves={waves}", flush=True)
    S, K, rb = 37, 8, 3072
    rng = np.random.default_rng(5)
    nrows = 300
    y = rng.integers(0, 2 ** 32, (nrows, rb // 4), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(0, nrows, (S, K)).astype(np.int32)
    rows[3, 0] = -1
    rows[36, 7] = -1
    want = np.zeros((S, rb // 4), np.uint32)
    for t in range(S):
        for k in range(K):
            if rows[t, k] >= 0:
                want[t] ^= y[rows[t, k]]
    y_d = torch.from_numpy(y.view(np.int32)).to(DEV)
    for kind in ("plain", "sc1"):
        out = torch.full((S, rb // 4), -1, dtype=torch.int32, device=DEV)
        pat.gather_persistent(y_d.view(torch.uint8), torch.from_numpy(rows).to(DEV), out.view(torch.uint8),
                              groups, waves, kind)()
        torch.cuda.synchronize()
        assert np.array_equal(_u32(out), want), kind


@pytest.mark.parametrize("policy", [0, 2, 3, 18, 19])
def test_gather_policy(pat, policy):
    print(f"case ceilings gather policy={policy}", flush=True)
    S, K, rb = 7, 8, 2048
    rng = np.random.default_rng(8)
    nrows = 60
    y = rng.integers(0, 2 ** 32, (nrows, rb // 4), dtype=np.uint64).astype(np.uint32)
    rows = rng.integers(0, nrows, (S, K)).astype(np.int32)
    rows[2, 6] = -1
    want = np.zeros((S, rb // 4), np.uint32)
    for t in range(S):
        for k in range(K):
            if rows[t, k] >= 0:
                want[t] ^= y[rows[t, k]]
    out = torch.full((S, rb // 4), -1, dtype=torch.int32, device=DEV)
    pat.gather_policy(torch.from_numpy(y.view(np.int32)).to(DEV).view(torch.uint8), torch.from_numpy(rows).to(DEV),
                      out.view(torch.uint8), policy)()
    torch.cuda.synchronize()
    assert np.array_equal(_u32(out), want)
