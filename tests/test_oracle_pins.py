"""Pins for the CPU oracle: each test ties it to something other than itself --
brute force, hand-worked examples, closed forms, invariants, or a library
routine that computes the same well-defined quantity.  All CPU-only.

Passages: expert parallelism with E/R local experts per rank and E divisible
by R (delect.ru glossary "Expert parallelism (EP)", DeepSpeed v0.14.5 example);
dispatch and combine as the activation exchange pair (same glossary,
MOELayer.forward; DeepEP analysis, "DeepEP introduction"); FP8 dispatch and
BF16 combine (DeepEP analysis, feature list and benchmark set-ups); zero-copy
writes to the final expert-grouped slot with static shapes (MoonEP article,
section 2); token_padding (MoonEP article, basic usage).
"""
import itertools
from fractions import Fraction

import numpy as np
import pytest
import torch

import oracle
from oracle import PAD_CAPACITY, PAD_MULTIPLE, PAD_NONE
from workloads import CONFIGS, make_workload

# ---------------------------------------------------------------------------
# helpers written independently of the oracle
# ---------------------------------------------------------------------------


def brute_layout(idx, E, R, pad_mode, pad_rows):
    """Direct O(N^2) statement of the layout: the row of entry i is the start of
    its expert's segment plus the number of earlier entries with the same expert;
    segment starts are sums over all lower expert ids."""
    flat = [int(v) for v in np.asarray(idx).reshape(-1)]
    n = len(flat)
    cnt = [sum(1 for v in flat if v == e) for e in range(E)]
    if pad_mode == PAD_NONE:
        seg = cnt[:]
    elif pad_mode == PAD_MULTIPLE:
        seg = [-(-c // pad_rows) * pad_rows for c in cnt]
    else:
        seg = [pad_rows] * E
    placed = [min(c, pad_rows) if pad_mode == PAD_CAPACITY else c for c in cnt]
    start = [sum(seg[:e]) for e in range(E)]
    pos = []
    for i, e in enumerate(flat):
        before = sum(1 for j in range(i) if flat[j] == e)
        pos.append(start[e] + before if before < placed[e] else -1)
    epr = E // R
    if pad_mode == PAD_MULTIPLE:
        rows = n + E * (pad_rows - 1)
    elif pad_mode == PAD_CAPACITY:
        rows = E * pad_rows
    else:
        rows = n
    src = [-1] * rows
    for i, p in enumerate(pos):
        if p >= 0:
            src[p] = i
    return dict(
        tokens_per_expert=placed,
        tokens_per_rank=[sum(placed[r * epr:(r + 1) * epr]) for r in range(R)],
        expert_offset=start + [sum(seg)],
        rank_offset=[start[r * epr] for r in range(R)] + [sum(seg)],
        pos=pos, src=src,
        status=int(any(c > pad_rows for c in cnt)) * 2 if pad_mode == PAD_CAPACITY else 0,
    )


def assert_layout_equal(lo, ref, shape):
    assert lo.tokens_per_expert.tolist() == ref["tokens_per_expert"]
    assert lo.tokens_per_rank.tolist() == ref["tokens_per_rank"]
    assert lo.expert_offset.tolist() == ref["expert_offset"]
    assert lo.rank_offset.tolist() == ref["rank_offset"]
    assert lo.pos.reshape(-1).tolist() == ref["pos"]
    assert lo.src.tolist() == ref["src"]
    assert int(lo.status[0]) == ref["status"]


def e4m3_table():
    """All 256 E4M3FN codes decoded from the format (1.4.3, bias 7, exponent 0
    subnormal, S.1111.111 NaN).  Written from the format, not the oracle."""
    vals = np.empty(256, np.float64)
    for c in range(256):
        s = -1.0 if c & 0x80 else 1.0
        e = (c >> 3) & 15
        m = c & 7
        if e == 15 and m == 7:
            vals[c] = np.nan
        elif e == 0:
            vals[c] = s * m * 2.0 ** -9
        else:
            vals[c] = s * (8 + m) * 2.0 ** (e - 10)
    return vals


def e4m3_bruteforce(v):
    """Nearest finite E4M3FN code by exhaustive search; ties to the code with a
    zero last mantissa bit; the sign of v is kept for zero results."""
    tab = e4m3_table()
    codes = np.arange(256)
    finite = ~np.isnan(tab)
    with np.errstate(invalid="ignore"):
        v = np.asarray(v, np.float64)
    out = np.empty(v.shape, np.uint8)
    fc, fv = codes[finite], tab[finite]
    for i, x in enumerate(v.reshape(-1)):
        if np.isnan(x):
            out.reshape(-1)[i] = 0x7F
            continue
        if np.isinf(x):
            out.reshape(-1)[i] = 0xFE if x < 0 else 0x7E
            continue
        # float64 distances are exact enough to order neighbours for |x| <= 2^40;
        # beyond every finite code the nearest one is the largest, so cap there
        xs = float(np.sign(x)) * min(abs(x), 2.0 ** 40)
        d = np.abs(fv - xs)
        best = d.min()
        cand = fc[d == best]
        # candidates: either one code, or a tie between two neighbours (+0/-0 also tie)
        if np.signbit(x):
            cand = [c for c in cand if c & 0x80 or tab[c] != 0.0] or list(cand)
        else:
            cand = [c for c in cand if not (c & 0x80)] or list(cand)
        if len(cand) > 1:
            even = [c for c in cand if (c & 1) == 0]
            cand = even
        out.reshape(-1)[i] = cand[0]
    return out


# ---------------------------------------------------------------------------
# layout
# ---------------------------------------------------------------------------


def test_layout_hand_example():
    """Worked by hand: S=3, K=2, E=4, R=2, rows grouped by expert, stable in t*K+k.
    idx = [[1,0],[1,3],[0,1]] -> counts [2,3,0,1]; starts [0,2,5,5]; the
    entries of expert 1 are (0,0),(1,0),(2,1) in that order -> rows 2,3,4."""
    idx = np.array([[1, 0], [1, 3], [0, 1]], np.int32)
    lo = oracle.layout(idx, E=4, R=2)
    assert lo.tokens_per_expert.tolist() == [2, 3, 0, 1]
    assert lo.expert_offset.tolist() == [0, 2, 5, 5, 6]
    assert lo.tokens_per_rank.tolist() == [5, 1]
    assert lo.rank_offset.tolist() == [0, 5, 6]
    assert lo.pos.tolist() == [[2, 0], [3, 5], [1, 4]]
    assert lo.src.tolist() == [1, 4, 0, 2, 5, 3]
    # padded to multiples of 4: segments 4,4,0,4
    lo = oracle.layout(idx, E=4, R=2, pad_mode=PAD_MULTIPLE, pad_rows=4)
    assert lo.expert_offset.tolist() == [0, 4, 8, 8, 12]
    assert lo.pos.tolist() == [[4, 0], [5, 8], [1, 6]]
    assert lo.src.tolist()[:12] == [1, 4, -1, -1, 0, 2, 5, -1, 3, -1, -1, -1]
    assert len(lo.src) == 6 + 4 * 3
    # capacity 2: expert 1's third entry (2,1) is not placed and flags overflow
    lo = oracle.layout(idx, E=4, R=2, pad_mode=PAD_CAPACITY, pad_rows=2)
    assert lo.expert_offset.tolist() == [0, 2, 4, 6, 8]
    assert lo.pos.tolist() == [[2, 0], [3, 6], [1, -1]]
    assert lo.tokens_per_expert.tolist() == [2, 2, 0, 1]
    assert int(lo.status[0]) == oracle.FLAG_CAPACITY


def test_layout_deepspeed_divisibility():
    """8 experts over 4 ranks: two local experts per rank; 8 over 3 is rejected."""
    rng = np.random.default_rng(1)
    idx = rng.integers(0, 8, size=(50, 2)).astype(np.int32)
    lo = oracle.layout(idx, E=8, R=4)
    cnt = np.bincount(idx.reshape(-1), minlength=8)
    assert lo.tokens_per_rank.tolist() == [int(cnt[0] + cnt[1]), int(cnt[2] + cnt[3]),
                                           int(cnt[4] + cnt[5]), int(cnt[6] + cnt[7])]
    assert lo.rank_offset.tolist() == [int(lo.expert_offset[2 * r]) for r in range(4)] + [100]
    with pytest.raises(ValueError):
        oracle.layout(idx, E=8, R=3)
    assert oracle.max_recv_rows(50, 2, 8, 3) == -1


@pytest.mark.parametrize("S,K,E,R", [(2, 2, 4, 2), (3, 2, 3, 3), (4, 2, 2, 1), (6, 1, 4, 4), (8, 1, 2, 2),
                                     (3, 3, 2, 2)])
@pytest.mark.parametrize("pad", [(PAD_NONE, 0), (PAD_MULTIPLE, 3), (PAD_CAPACITY, 2)])
def test_layout_exhaustive_tiny(S, K, E, R, pad):
    """Every routing in [0,E)^(S*K) for tiny shapes, against the brute force."""
    n = S * K
    for combo in itertools.product(range(E), repeat=n):
        idx = np.array(combo, np.int32).reshape(S, K)
        lo = oracle.layout(idx, E, R, *pad)
        assert_layout_equal(lo, brute_layout(idx, E, R, *pad), (S, K))


@pytest.mark.parametrize("seed", range(6))
def test_layout_random_vs_bruteforce(seed):
    rng = np.random.default_rng(100 + seed)
    S = int(rng.integers(0, 40))
    K = int(rng.integers(1, 5))
    R = int(rng.choice([1, 2, 4]))
    E = R * int(rng.integers(1, 5))
    pad = [(PAD_NONE, 0), (PAD_MULTIPLE, int(rng.integers(1, 6))), (PAD_CAPACITY, int(rng.integers(1, 12)))][seed % 3]
    idx = rng.integers(0, E, size=(S, K)).astype(np.int32)
    lo = oracle.layout(idx, E, R, *pad)
    assert_layout_equal(lo, brute_layout(idx, E, R, *pad), (S, K))


def check_layout_invariants(lo, idx, E, R, pad_mode, pad_rows):
    flat = idx.reshape(-1)
    n = flat.size
    pos = lo.pos.reshape(-1)
    cnt = np.bincount(flat[(flat >= 0) & (flat < E)], minlength=E)
    placed = np.minimum(cnt, pad_rows) if pad_mode == PAD_CAPACITY else cnt
    # counts sum to S*K (no capacity drops), each placed entry exactly once
    assert lo.tokens_per_expert.tolist() == placed.tolist()
    if pad_mode != PAD_CAPACITY:
        assert int(lo.tokens_per_expert.sum()) == n
    ok = pos >= 0
    assert np.all(lo.src[pos[ok]] == np.nonzero(ok)[0])
    assert int((lo.src >= 0).sum()) == int(ok.sum())
    # segment offsets are the scan of the (padded) counts
    seg = np.diff(lo.expert_offset)
    if pad_mode == PAD_NONE:
        assert np.array_equal(seg, cnt)
    elif pad_mode == PAD_MULTIPLE:
        assert np.all(seg % pad_rows == 0) and np.all(seg >= cnt) and np.all(seg - cnt < pad_rows)
    else:
        assert np.all(seg == pad_rows)
    assert lo.expert_offset[0] == 0
    # rows stay inside their expert's segment, increasing in t*K+k
    for e in range(E):
        sel = np.nonzero((flat == e) & ok)[0]
        p = pos[sel]
        assert np.all(np.diff(p) == 1)
        if sel.size:
            assert p[0] == lo.expert_offset[e]
    epr = E // R
    assert lo.rank_offset.tolist() == [int(lo.expert_offset[r * epr]) for r in range(R)] + [int(lo.expert_offset[E])]
    assert lo.tokens_per_rank.tolist() == [int(placed[r * epr:(r + 1) * epr].sum()) for r in range(R)]


@pytest.mark.parametrize("name", list(CONFIGS))
def test_layout_invariants_configs(name):
    cfg = CONFIGS[name]
    w = make_workload(cfg, with_hidden=False)
    lo = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    check_layout_invariants(lo, w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    assert int(lo.status[0]) == 0


def test_layout_bad_ids_flagged():
    idx = np.array([[0, 5], [-1, 1], [2, 2]], np.int32)
    lo = oracle.layout(idx, E=4, R=2)
    assert lo.pos.tolist() == [[0, -1], [-1, 1], [2, 3]]
    assert int(lo.status[0]) == oracle.FLAG_BAD_EXPERT
    assert lo.tokens_per_expert.tolist() == [1, 1, 2, 0]


# ---------------------------------------------------------------------------
# number formats
# ---------------------------------------------------------------------------


def test_e4m3_decode_matches_format_table():
    tab = e4m3_table()
    got = np.array([oracle.f32_from_e4m3(c) for c in range(256)], np.float64)
    assert np.array_equal(np.isnan(got), np.isnan(tab))
    assert np.array_equal(got[~np.isnan(tab)], tab[~np.isnan(tab)])
    assert tab[0x7E] == 448.0 and tab[0x01] == 2.0 ** -9 and tab[0x08] == 2.0 ** -6


def _e4m3_sweep_values():
    bf = np.arange(65536, dtype=np.uint32) << 16
    allbf = bf.view(np.float32)
    tab = e4m3_table()
    fin = np.sort(np.unique(np.abs(tab[~np.isnan(tab)])))
    mids = ((fin[:-1] + fin[1:]) / 2).astype(np.float32)
    mids = np.concatenate([mids, np.float32([464.0])])
    near = np.concatenate([mids, np.nextafter(mids, np.float32(np.inf)), np.nextafter(mids, np.float32(0))])
    near = np.concatenate([near, -near])
    rng = np.random.default_rng(7)
    rnd = (rng.choice([-1, 1], 20000) * np.exp(rng.uniform(np.log(1e-4), np.log(600), 20000))).astype(np.float32)
    return np.concatenate([allbf, near, rnd, np.float32([0.0, -0.0, np.inf, -np.inf, 1e-40, -1e-40])])


def test_e4m3_encode_vs_bruteforce():
    """RNE with ties to even and saturation, against exhaustive nearest-code search:
    every bf16 pattern, every midpoint between neighbouring codes and one fp32 ulp
    either side, and random magnitudes from 1e-4 to 600."""
    v = _e4m3_sweep_values()
    got = oracle.e4m3_from_f32_array(v)
    ref = e4m3_bruteforce(v)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(v[i]), int(got[i]), int(ref[i])) for i in bad[:10]]


def test_e4m3_encode_vs_torch_cast():
    """torch's float8_e4m3fn cast rounds to nearest even and agrees with the
    saturating encoder wherever it does not overflow (|v| < 464)."""
    v = _e4m3_sweep_values()
    v = v[np.isfinite(v) & (np.abs(v) < 464)]
    t = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(oracle.e4m3_from_f32_array(v), t)


def test_bf16_round_vs_torch():
    rng = np.random.default_rng(3)
    v = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e36).astype(np.float32),
        (rng.standard_normal(20000) * 1e-39).astype(np.float32),   # fp32 subnormals
        np.float32([3.3895314e38, 3.3961776e38, 3.4028235e38, np.inf, -np.inf, 0.0, -0.0]),
    ])
    # exact ties: bf16 value plus half a bf16 ulp
    b = rng.integers(0, 0x7F7F, 20000).astype(np.uint32) << 16
    ties = (b | 0x8000).view(np.float32)
    v = np.concatenate([v, ties, -ties])
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_from_f32_array(v), ref)
    assert oracle.bf16_from_f32(float("nan")) == 0x7FC0


# ---------------------------------------------------------------------------
# FP8 quantisation
# ---------------------------------------------------------------------------


def test_fp8_row_invariants_and_error_bound():
    w = make_workload(CONFIGS["decode"])
    tab = e4m3_table()
    for t in range(0, w.cfg.S, 7):
        row = w.hidden[t]
        codes, scales = oracle.quantize_row_fp8(row)
        x = (row.astype(np.uint32) << 16).view(np.float32).astype(np.float64).reshape(-1, 128)
        c = codes.reshape(-1, 128)
        for b in range(x.shape[0]):
            amax = np.abs(x[b]).max()
            assert scales[b] > 0
            # the largest-magnitude element encodes +-448
            j = int(np.argmax(np.abs(x[b])))
            assert c[b, j] in (0x7E, 0xFE)
            # dequantisation error bound: half a step of the e4m3 grid at |x/scale|
            q = x[b] / float(scales[b])
            deq = tab[c[b]]
            step = np.where(np.abs(q) >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(np.abs(q), 2.0 ** -6))) - 3),
                            2.0 ** -9)
            # (the encoder sees the fp32 quotient, off the exact one by <= |q| 2^-24)
            assert np.all(np.abs(deq - q) <= step / 2 + np.abs(q) * 2.0 ** -23)
            assert np.all(np.sign(deq[deq != 0]) == np.sign(q[deq != 0]))
            assert abs(float(scales[b]) * 448.0 - amax) <= amax * 2.0 ** -23


def test_fp8_scale_one_block_is_plain_cast():
    """A block whose amax is 448 has scale exactly 1, so its codes are the plain
    e4m3 cast of its values (checked against the brute force)."""
    rng = np.random.default_rng(5)
    x = (rng.standard_normal(128) * 60).astype(np.float32)
    x[17] = -448.0
    row = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    codes, scales = oracle.quantize_row_fp8(row)
    assert scales[0] == 1.0
    xv = (row.astype(np.uint32) << 16).view(np.float32)
    assert np.array_equal(codes, e4m3_bruteforce(xv))


def test_fp8_zero_block_and_sign_symmetry():
    row = np.zeros(256, np.uint16)
    row[128:] = 0x3F80  # 1.0
    row[200] = 0xC000   # -2.0
    codes, scales = oracle.quantize_row_fp8(row)
    assert scales[0] == 0.0 and np.all(codes[:128] == 0)
    neg = row ^ np.uint16(0x8000)
    ncodes, nscales = oracle.quantize_row_fp8(neg)
    assert np.array_equal(nscales, scales)
    assert np.array_equal(ncodes[128:], codes[128:] ^ 0x80)
    assert np.all(ncodes[:128] == 0)   # all-zero block (now -0.0) still gives 0x00


# Exact rational arithmetic: the correctly rounded fp32 result of an operation
# is the fp32 value nearest its exact value (ties to the even significand).
# Written from the IEEE 754 definition, independent of any float hardware.


def f32_nearest(r: Fraction) -> Fraction:
    """Nearest fp32 value to the exact rational r (normal range), ties to even."""
    if r == 0:
        return Fraction(0)
    sign = -1 if r < 0 else 1
    a = abs(r)
    e = a.numerator.bit_length() - a.denominator.bit_length()
    if Fraction(2) ** e > a:
        e -= 1
    assert Fraction(2) ** e <= a < Fraction(2) ** (e + 1) and -126 <= e <= 127
    ulp = Fraction(2) ** (e - 23)
    n, rem = divmod(a, ulp)
    if rem * 2 > ulp or (rem * 2 == ulp and n % 2 == 1):
        n += 1
    return sign * n * ulp


def e4m3_nearest_exact(r: Fraction) -> int:
    """E4M3FN code of the exact rational r: the nearest finite code value, ties
    to the even mantissa, saturating at +-448, the sign of r kept."""
    sign = 0x80 if r < 0 else 0x00
    a = abs(r)
    best = None
    for c in range(0x7F):                       # 0x00..0x7E: every finite magnitude
        e, m = c >> 3, c & 7
        v = Fraction(m, 512) if e == 0 else Fraction(8 + m, 8) * Fraction(2) ** (e - 7)
        d = abs(v - a)
        if best is None or d < best[0] or (d == best[0] and c % 2 == 0):
            best = (d, c)
    return sign | best[1]


def _f32_exact(v) -> Fraction:
    return Fraction(float(np.float32(v)))


def test_fp8_hand_block_scale_and_quotient_rounding():
    """One block where the readings of the quantiser give different bits.

    amax = 1.53125 (bf16 0x3FC4) = 49/32, so amax/448 = 7/2048 exactly; amax
    times a rounded 1/448 lands one fp32 step above it.  The element
    x = 0.0247802734375 (bf16 0x3CCB) divided by the exact scale gives 7.25,
    exactly halfway between the E4M3 values 7.0 and 7.5, so the tie goes to
    the even mantissa: 7.0, code 0x4E.  x times a rounded 448/amax, or times a
    rounded 1/scale, gives 7.25 + 2^-21, past the midpoint: 7.5, code 0x4F.
    Expected bits come from exact rational arithmetic only; the other readings
    are asserted to differ so the case stays discriminating."""
    amax_bits, x_bits = 0x3FC4, 0x3CCB
    amax = Fraction(1.53125)
    x = Fraction(0.0247802734375)
    assert _f32_exact((np.uint32(amax_bits) << 16).view(np.float32)) == amax
    assert _f32_exact((np.uint32(x_bits) << 16).view(np.float32)) == x
    scale = f32_nearest(amax / 448)
    q = f32_nearest(x / scale)
    code_x = e4m3_nearest_exact(q)
    # the alternative readings, each step rounded to fp32
    scale_recip = f32_nearest(amax * f32_nearest(Fraction(1, 448)))
    q_mul448 = f32_nearest(x * f32_nearest(448 / amax))
    q_recip = f32_nearest(x * f32_nearest(1 / scale))
    assert scale_recip != scale
    assert e4m3_nearest_exact(q_mul448) != code_x and e4m3_nearest_exact(q_recip) != code_x
    assert scale == Fraction(7, 2048) and q == Fraction(29, 4)
    assert code_x == 0x4E                       # 7.0 = 2^2 * (1 + 6/8)

    row = np.zeros(256, np.uint16)
    row[3], row[40], row[77] = amax_bits, x_bits, x_bits | 0x8000
    row[128 + 5] = 0xBFC4                       # second block: amax from a negative value
    row[128 + 6] = x_bits
    codes, scales = oracle.quantize_row_fp8(row)
    assert Fraction(float(scales[0])) == scale and Fraction(float(scales[1])) == scale
    assert codes[3] == 0x7E and codes[128 + 5] == 0xFE
    assert codes[40] == code_x and codes[77] == (code_x | 0x80) and codes[128 + 6] == code_x
    others = np.ones(256, bool)
    others[[3, 40, 77, 128 + 5, 128 + 6]] = False
    assert np.all(codes[others] == 0x00)


def e4m3_nearest_vec(v: np.ndarray) -> np.ndarray:
    """Vectorised exhaustive search: for each value, the nearest of the 127
    finite non-negative code magnitudes to |v| (ties to the even mantissa), with
    v's sign bit set on the code.  Distances in float64 are exact here
    (|v| <= 2^9, every code and every fp32 input is a short dyadic rational)."""
    tab = e4m3_table()[:0x7F]
    v = np.asarray(v, np.float32)
    a = np.abs(v).astype(np.float64)
    out = np.empty(a.shape, np.uint8)
    flat_a, flat_o = a.reshape(-1), out.reshape(-1)
    for i in range(0, flat_a.size, 1 << 15):
        d = np.abs(tab[None, :] - flat_a[i:i + (1 << 15), None])
        best = d.min(axis=1, keepdims=True)
        hit = d == best
        n_hit = hit.sum(axis=1)
        first = hit.argmax(axis=1)
        # a tie is between two neighbouring codes: keep the even one
        pick = np.where((n_hit > 1) & (first % 2 == 1), first + 1, first)
        flat_o[i:i + (1 << 15)] = pick
    return out | np.where(np.signbit(v), 0x80, 0x00).astype(np.uint8)


@pytest.mark.parametrize("name,tokens", [("decode", 128), ("prefill", 512)])
def test_fp8_codes_and_scales_vs_numpy_division(name, tokens):
    """Every block of the decode batch and of 512 prefill tokens, recomputed
    outside the oracle: the scale is numpy's IEEE fp32 quotient amax / 448, each
    code the exhaustive nearest-code search applied to numpy's fp32 quotient
    x / scale.  Codes and scale bits must be identical."""
    cfg = CONFIGS[name]
    hid = make_workload(cfg).hidden[:tokens]
    x = (hid.astype(np.uint32) << 16).view(np.float32).reshape(tokens, -1, 128)
    amax = np.abs(x).max(axis=2)
    assert np.all(amax > 0)
    scale = amax / np.float32(448.0)
    assert scale.dtype == np.float32
    q = x / scale[:, :, None]
    assert q.dtype == np.float32
    want_codes = e4m3_nearest_vec(q).reshape(tokens, -1)
    for t in range(tokens):
        codes, scales = oracle.quantize_row_fp8(hid[t])
        assert np.array_equal(scales.view(np.uint32), scale[t].view(np.uint32)), t
        assert np.array_equal(codes, want_codes[t]), t


# ---------------------------------------------------------------------------
# combine
# ---------------------------------------------------------------------------


def _bf16_to_f64(bits):
    return (np.asarray(bits).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def test_combine_fma_chain_order_pins():
    """Hand-worked cases where the rounding of the fp32 chain decides the bf16 bit.
    (a) terms 1+2^-8, then 0x1.fc07f2p-25 * (1+2^-7) (exact product just above
        2^-24, rounds to 2^-24 on its own): a fused chain in ascending k lands
        above the fp32 midpoint -> 1+2^-8+2^-23 -> bf16 0x3F81; an unfused
        multiply-add or the reverse order ties to 1+2^-8 -> bf16 0x3F80.
    (b) terms 1+2^-8, 3*2^-26, 3*2^-26: ascending order absorbs each small term
        (0.375 ulp) -> bf16 tie -> 0x3F80; descending sums them first (0.75 ulp)
        -> 0x3F81."""
    y = np.array([[0x3F80], [0x3F81], [0x3F80]], np.uint16)       # 1.0, 1+2^-7, 1.0
    pos = np.array([[0, 1]], np.int32)
    w = np.array([[1 + 2 ** -8, float.fromhex("0x1.fc07f2p-25")]], np.float32)
    assert oracle.combine(y, pos, w).tolist() == [[0x3F81]]
    pos3 = np.array([[0, 2, 2]], np.int32)
    w3 = np.array([[1 + 2 ** -8, 3 * 2 ** -26, 3 * 2 ** -26]], np.float32)
    assert oracle.combine(y, pos3, w3).tolist() == [[0x3F80]]


def test_combine_shared_added_after_chain():
    """Shared output added after the routed fma chain, not used as its start.

    Terms w0*y0 = 2^-8 + 3*2^-26 and w1*y1 = 3*2^-26 (y = 1.0), shared = 1.0.
    Routed chain first: the two small parts meet at the scale of 2^-8 and sum
    exactly to 2^-8 + 6*2^-26; adding 1.0 then leaves 0.75 of an fp32 step at 1
    past 1 + 2^-8, which rounds up to 1 + 2^-8 + 2^-23, above the bf16 midpoint:
    bf16 1 + 2^-7 = 0x3F81.  Starting the chain from the shared 1.0 instead,
    each small part is 0.375 of a step and is absorbed, leaving exactly the
    midpoint 1 + 2^-8, which ties to the even bf16 1.0 = 0x3F80."""
    y = np.array([[0x3F80], [0x3F80]], np.uint16)
    pos = np.array([[0, 1]], np.int32)
    w = np.array([[2 ** -8 + 3 * 2 ** -26, 3 * 2 ** -26]], np.float32)
    assert float(w[0, 0]) == 2 ** -8 + 3 * 2 ** -26 and float(w[0, 1]) == 3 * 2 ** -26
    shared = np.array([[0x3F80]], np.uint16)
    # the two orders, every step rounded to fp32 in exact arithmetic
    t0, t1, one = Fraction(float(w[0, 0])), Fraction(float(w[0, 1])), Fraction(1)
    last = f32_nearest(f32_nearest(f32_nearest(t0) + t1) + one)
    first = f32_nearest(f32_nearest(one + t0) + t1)
    assert last == 1 + Fraction(1, 256) + Fraction(1, 2 ** 23) and first == 1 + Fraction(1, 256)
    assert oracle.combine(y, pos, w, shared).tolist() == [[0x3F81]]
    # without the shared output the chain alone is 2^-8 + 6*2^-26 -> bf16 2^-8
    assert oracle.combine(y, pos, w).tolist() == [[0x3B80]]


@pytest.mark.parametrize("name", ["tiny", "dsmoe16b"])
def test_combine_round_trip_identity(name):
    """combine(dispatch(x)) with identity experts and weights summing to 1 gives x
    back bit for bit: the fp32 chain is within ~K*2^-23 relative of x, far inside
    half a bf16 step.  Without weights the result is bf16(K*x), exact in fp32."""
    cfg = CONFIGS[name]
    w = make_workload(cfg)
    if name == "dsmoe16b":   # keep the CPU test short: first 2048 tokens
        w.hidden, w.topk_idx, w.topk_w = w.hidden[:2048], w.topk_idx[:2048], w.topk_w[:2048]
    lo = oracle.layout(w.topk_idx, cfg.E, cfg.R)
    recv, recv_w = oracle.dispatch_bf16(w.hidden, lo.pos, len(lo.src), w.topk_w)
    assert np.array_equal(recv_w[lo.pos.reshape(-1)], w.topk_w.reshape(-1))
    out = oracle.combine(recv, lo.pos, w.topk_w)
    # the chain starts from +0.0, so an input -0.0 comes back as +0.0
    assert np.array_equal(out, np.where((w.hidden & 0x7FFF) == 0, 0, w.hidden))
    out1 = oracle.combine(recv, lo.pos, None)
    kx = torch.from_numpy((_bf16_to_f64(w.hidden) * cfg.K + 0.0).astype(np.float32))
    kx = kx.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(out1, np.where((kx & 0x7FFF) == 0, 0, kx))


def test_combine_one_hot_and_shared_only():
    cfg = CONFIGS["tiny"]
    w = make_workload(cfg)
    lo = oracle.layout(w.topk_idx, cfg.E, cfg.R)
    y = oracle.dispatch_bf16(w.hidden, lo.pos, len(lo.src))[0]
    rng = np.random.default_rng(9)
    y = rng.integers(0, 0x7F00, y.shape).astype(np.uint16) ^ (rng.integers(0, 2, y.shape).astype(np.uint16) << 15)
    j = rng.integers(0, cfg.K, cfg.S)
    onehot = np.zeros((cfg.S, cfg.K), np.float32)
    onehot[np.arange(cfg.S), j] = 1.0
    out = oracle.combine(y, lo.pos, onehot)
    sel = y[lo.pos[np.arange(cfg.S), j]]
    # +0.0 + (+-0.0) gives +0.0; all other values come back unchanged
    sel = np.where((sel & 0x7FFF) == 0, 0, sel)
    assert np.array_equal(out, sel)
    shared = make_workload(cfg, seed=77).hidden
    zero = np.zeros((cfg.S, cfg.K), np.float32)
    y_finite = np.where((y & 0x7F80) == 0x7F80, 0, y).astype(np.uint16)
    assert np.array_equal(oracle.combine(y_finite, lo.pos, zero, shared),
                          np.where((shared & 0x7FFF) == 0, 0, shared))


def test_combine_random_within_fp64_bound():
    """Against the exact sum in float64: |out - exact| <= half a bf16 step at the
    result + K * 2^-24 * sum|w*y| (the fp32 fma chain's error) + shared term."""
    cfg = CONFIGS["dsmoe16b"]
    w = make_workload(cfg)
    S = 512
    idx, tw, shared = w.topk_idx[:S], w.topk_w[:S], w.shared[:S]
    lo = oracle.layout(idx, cfg.E, cfg.R)
    y = np.random.default_rng(11).standard_normal((len(lo.src), cfg.H)).astype(np.float32)
    y = torch.from_numpy(y).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    out = oracle.combine(y, lo.pos, tw, shared)
    yv = _bf16_to_f64(y)
    terms = tw.astype(np.float64)[:, :, None] * yv[lo.pos]          # [S,K,H]
    exact = terms.sum(axis=1) + _bf16_to_f64(shared)
    got = _bf16_to_f64(out)
    bound = (np.abs(exact) * 2.0 ** -8 + cfg.K * 2.0 ** -23 * (np.abs(terms).sum(axis=1) + np.abs(_bf16_to_f64(shared)))
             + 1e-30)
    assert np.all(np.abs(got - exact) <= bound)
    # a dropped term or a flipped sign is far outside that bound
    bad = terms[:, 1:].sum(axis=1) + _bf16_to_f64(shared)
    assert np.mean(np.abs(got - bad) > bound) > 0.5


def test_fp8_round_trip_combine_bound():
    """FP8 dispatch, identity-dequant experts, weighted combine: each output is
    within the e4m3 quantisation bound (half a grid step times the scale) plus
    half a bf16 step of the token's value."""
    cfg = CONFIGS["decode"]
    w = make_workload(cfg)
    lo = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    recv, scales, _ = oracle.dispatch_fp8(w.hidden, lo.pos, len(lo.src))
    y = oracle.dequant_identity_expert(recv, scales)
    out = oracle.combine(y, lo.pos, w.topk_w)
    x = _bf16_to_f64(w.hidden)
    sc = np.stack([oracle.quantize_row_fp8(w.hidden[t])[1] for t in range(cfg.S)])   # [S, H/128]
    assert sc.shape[1] == cfg.H // 128
    scale = np.repeat(sc.astype(np.float64), 128, axis=1)
    q = np.abs(x) / scale
    # half a step of the e4m3 grid at q: 2^(floor(log2 q) - 4) for normals, 2^-10 below 2^-6
    half_step = np.where(q >= 2.0 ** -6, 2.0 ** (np.floor(np.log2(np.maximum(q, 2.0 ** -6))) - 4), 2.0 ** -10)
    got = _bf16_to_f64(out)
    # plus two bf16 roundings (the expert output and the combine result)
    bound = scale * half_step * 1.001 + np.abs(x) * 2.0 ** -7 + 1e-30
    assert np.all(np.abs(got - x) <= bound)


# ---------------------------------------------------------------------------
# generators (input recipes)
# ---------------------------------------------------------------------------


def test_generator_properties():
    c2 = CONFIGS["prefill"]
    w2 = make_workload(c2, with_hidden=False)
    ranks = w2.topk_idx // (c2.E // c2.R)
    assert max(len(set(r)) for r in ranks.tolist()) <= 4          # top-4 groups = ranks
    for cfg_name in CONFIGS:
        cfg = CONFIGS[cfg_name]
        w = make_workload(cfg, with_hidden=False)
        assert all(len(set(r)) == cfg.K for r in w.topk_idx.tolist())   # distinct experts
        assert np.all((w.topk_idx >= 0) & (w.topk_idx < cfg.E))
        assert np.allclose(w.topk_w.astype(np.float64).sum(axis=1), 1.0, atol=1e-6)
    from workloads import maxvio
    c4 = CONFIGS["skew"]
    w4 = make_workload(c4, with_hidden=False)
    assert abs(maxvio(w4.topk_idx, c4.E) - 20.0) <= 0.5
    assert int(np.bincount(w4.topk_idx.reshape(-1)).argmax()) == 0   # hottest expert is 0


# ---------------------------------------------------------------------------
# balanced layout (redundant expert slots)
# ---------------------------------------------------------------------------


def test_balanced_hand_example():
    """Worked by hand: E=4 experts on R=2 ranks, B=1 slot, counts [5,1,1,1],
    N=8 so each rank's quota is 4.  Rank 0 holds 6 (surplus 2), rank 1 holds 2.
    Expert 0 (rank 0's largest) sheds 2 entries into rank 1's slot 0.  Its
    entries are t = 0,1,3,5,7: the first three stay home (rows 0..2), t=5 and 7
    go to the replica (rows 6, 7).  Rows: rank 0 = [e0 x3, e1], rank 1 = [e2,
    e3, slot0: e0 x2]."""
    idx = np.array([[0], [0], [1], [0], [2], [0], [3], [0]], np.int32)
    lo = oracle.layout_balanced(idx, 4, 2, 1)
    assert lo.tokens_per_rank.tolist() == [4, 4]
    assert lo.seg_offset.tolist() == [0, 3, 4, 4, 5, 6, 8]
    assert lo.slot_expert.tolist() == [-1, 0]
    assert lo.pos.reshape(-1).tolist() == [0, 1, 3, 2, 4, 6, 5, 7]
    assert lo.expert_offset.tolist() == [0, 3, 4, 5, 8]
    assert int(lo.status[0]) == 0


def test_balanced_hand_example_two_destinations():
    """E=4, R=4 (one expert per rank), B=2, counts [9,1,1,1] (N=12, quota 3):
    expert 0 sheds 6: rank 1 takes 2, rank 2 takes 2, rank 3 takes 2 (lowest
    destination first, each as much as its room).  Not enough slots with B=0:
    nothing moves and the layout is flagged."""
    idx = np.array([0] * 9 + [1, 2, 3], np.int32).reshape(12, 1)
    lo = oracle.layout_balanced(idx, 4, 4, 2)
    assert lo.tokens_per_rank.tolist() == [3, 3, 3, 3]
    assert lo.slot_expert.tolist() == [-1, -1, 0, -1, 0, -1, 0, -1]
    # expert 0's entries 0..8: rows 0,1,2 home; 3,4 -> rank1 slot0 (rows 4,5); 5,6 -> rank2; 7,8 -> rank3
    assert lo.pos.reshape(-1).tolist()[:9] == [0, 1, 2, 4, 5, 7, 8, 10, 11]
    lo0 = oracle.layout_balanced(idx, 4, 4, 0)
    assert int(lo0.status[0]) == oracle.FLAG_UNBALANCED
    assert lo0.pos.reshape(-1).tolist() == oracle.layout(idx, 4, 4).pos.reshape(-1).tolist()


def check_balanced(lo, idx, E, R, B):
    flat = idx.reshape(-1)
    n = flat.size
    pos = lo.pos.reshape(-1)
    ok = (flat >= 0) & (flat < E)
    valid = int(ok.sum())
    epr, nseg = E // R, E // R + B
    # every valid entry exactly once, rows [0, valid) all used
    assert np.all(pos[~ok] == -1)
    assert np.all(lo.src[pos[ok]] == np.nonzero(ok)[0])
    assert sorted(pos[ok].tolist()) == list(range(valid))
    assert np.all(lo.src[valid:] == -1)
    seg = np.diff(lo.seg_offset)
    assert lo.seg_offset[0] == 0 and lo.seg_offset[-1] == valid
    quota = [valid // R + (1 if r < valid % R else 0) for r in range(R)]
    cnt = np.bincount(flat[ok], minlength=E)
    load = [int(cnt[r * epr:(r + 1) * epr].sum()) for r in range(R)]
    assert lo.tokens_per_expert.tolist() == cnt.tolist()
    balanced = not (int(lo.status[0]) & oracle.FLAG_UNBALANCED)
    for r in range(R):
        rows = int(lo.seg_offset[(r + 1) * nseg] - lo.seg_offset[r * nseg])
        assert lo.tokens_per_rank[r] == rows
        assert lo.rank_offset[r] == lo.seg_offset[r * nseg]
        if balanced:
            assert rows == quota[r]
        # a rank above its quota only sheds, a rank below only receives
        used = [s for s in range(B) if lo.slot_expert[r * B + s] >= 0]
        assert used == list(range(len(used)))        # slots fill in order
        if used:
            assert load[r] < quota[r]
            assert rows <= quota[r]
        for s in range(B):
            e = lo.slot_expert[r * B + s]
            if e >= 0:
                assert e // epr != r                  # never a replica on the owner
                assert seg[r * nseg + epr + s] > 0
            else:
                assert seg[r * nseg + epr + s] == 0
    # each segment holds entries of one expert; per expert the rows follow t*K+k:
    # home segment first, then replicas in ascending destination rank
    seg_of_row = np.searchsorted(lo.seg_offset, np.arange(valid), side="right") - 1
    for e in range(E):
        ent = np.nonzero(flat == e)[0]
        rows = pos[ent]
        segs = seg_of_row[rows]
        home_seg = (e // epr) * nseg + e % epr
        order = [home_seg] + [r * nseg + epr + s for r in range(R) for s in range(B)
                              if lo.slot_expert[r * B + s] == e]
        expect = np.concatenate([np.arange(lo.seg_offset[g], lo.seg_offset[g + 1]) for g in order])
        assert rows.tolist() == expect.tolist()
        assert set(segs.tolist()) <= set(order)
        # a shed expert: its rank sheds from its largest experts first
    for r in range(R):
        experts = list(range(r * epr, (r + 1) * epr))
        shed = [e for e in experts if lo.expert_offset[e] >= 0 and
                (lo.seg_offset[(e // epr) * nseg + e % epr + 1] - lo.seg_offset[(e // epr) * nseg + e % epr]) < cnt[e]]
        by_size = sorted(experts, key=lambda e: (-cnt[e], e))
        assert shed == sorted(by_size[:len(shed)])     # the shed set is a prefix of the size order
    if B == 0 or R == 1:
        assert pos.tolist() == oracle.layout(idx, E, R).pos.reshape(-1).tolist()


@pytest.mark.parametrize("seed", range(8))
def test_balanced_random_invariants(seed):
    rng = np.random.default_rng(500 + seed)
    R = int(rng.choice([1, 2, 4, 8]))
    E = R * int(rng.integers(1, 9))
    S, K = int(rng.integers(0, 200)), int(rng.integers(1, 5))
    B = int(rng.integers(0, 5))
    p = rng.random(E) ** 3                       # skewed expert popularity
    idx = rng.choice(E, size=(S, K), p=p / p.sum()).astype(np.int32)
    if seed % 3 == 0 and idx.size:
        idx.reshape(-1)[rng.integers(0, idx.size, 3)] = -1
    lo = oracle.layout_balanced(idx, E, R, B)
    check_balanced(lo, idx, E, R, B)


@pytest.mark.parametrize("E,R,B", [(4, 2, 1), (4, 4, 1), (6, 3, 2)])
def test_balanced_exhaustive_tiny(E, R, B):
    S, K = 5, 1
    for combo in itertools.product(range(E), repeat=S * K):
        idx = np.array(combo, np.int32).reshape(S, K)
        check_balanced(oracle.layout_balanced(idx, E, R, B), idx, E, R, B)


def test_balanced_already_even_is_plain_layout():
    """Loads already at quota: nothing moves, rows equal the plain layout's."""
    idx = np.tile(np.arange(8, dtype=np.int32), (6, 1))       # every expert 6 entries
    lo = oracle.layout_balanced(idx, 8, 4, 3)
    assert np.all(lo.slot_expert == -1)
    assert lo.pos.tolist() == oracle.layout(idx, 8, 4).pos.tolist()


def test_balanced_skew_config():
    """The skewed workload (maxvio 20, rank 0 holding 4.3x its quota): with 16
    slots per rank every rank gets exactly S*K/R = 4096 rows; with 8 slots the
    planner runs out of room on the last destination and flags it."""
    cfg = CONFIGS["skew"]
    w = make_workload(cfg, with_hidden=False)
    lo = oracle.layout_balanced(w.topk_idx, cfg.E, cfg.R, 16)
    assert int(lo.status[0]) == 0
    assert lo.tokens_per_rank.tolist() == [cfg.S * cfg.K // cfg.R] * cfg.R
    check_balanced(lo, w.topk_idx, cfg.E, cfg.R, 16)
    lo8 = oracle.layout_balanced(w.topk_idx, cfg.E, cfg.R, 8)
    assert int(lo8.status[0]) == oracle.FLAG_UNBALANCED
    check_balanced(lo8, w.topk_idx, cfg.E, cfg.R, 8)


def test_zero_padding_hand_example():
    src = np.array([0, -1, 2, -1], np.int32)
    rng = np.random.default_rng(3)
    recv = rng.integers(1, 255, (4, 16)).astype(np.uint8)
    scales = rng.random((4, 2)).astype(np.float32) + 1.0
    out, sc = oracle.zero_padding(src, recv, scales)
    assert np.array_equal(out[[0, 2]], recv[[0, 2]]) and np.array_equal(sc[[0, 2]], scales[[0, 2]])
    assert not out[[1, 3]].any() and not sc[[1, 3]].any()
    out16, none = oracle.zero_padding(src, recv.view(np.uint16))     # bf16 rows, no scales
    assert none is None and np.array_equal(out16.view(np.uint8)[[0, 2]], recv[[0, 2]])
    assert not out16[[1, 3]].any()


def test_zero_padding_after_padded_dispatch():
    """On a capacity-padded layout, after zero padding every receive row either
    holds the codes of the token its src names or is all zero (codes and scale)."""
    cfg = CONFIGS["decode"]
    w = make_workload(cfg)
    lo = oracle.layout(w.topk_idx, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
    rows = len(lo.src)
    codes, scales, _ = oracle.dispatch_fp8(w.hidden, lo.pos, rows)
    codes[lo.src < 0] = 0xA5                         # stale bytes where nothing was written
    scales[lo.src < 0] = 7.0
    zc, zs = oracle.zero_padding(lo.src, codes, scales)
    pad = lo.src < 0
    assert pad.sum() == rows - cfg.S * cfg.K
    assert not zc[pad].any() and not zs[pad].any()
    q = np.stack([oracle.quantize_row_fp8(w.hidden[t])[0] for t in range(cfg.S)])
    assert np.array_equal(zc[~pad], q[lo.src[~pad] // cfg.K])
