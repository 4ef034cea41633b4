"""Seeded input recipes for the five MoE expert-parallel workloads.

Every array comes from numpy's PCG64 generator, seeded through a
``SeedSequence([seed, tag])`` with one tag per tensor, so that a tensor does
not change when another one is added or resized.  fp32 -> bf16 conversion of
drawn values uses torch's own cast (round to nearest even); that is a library
routine used only to store inputs, never the path's arithmetic.

Workload shapes (DeepEP deep-analysis article, "performance" section: 4096
tokens per batch, hidden 7168, top-4 groups / top-8 experts for the normal
kernels, 128 tokens for the low-latency kernels; DeepSeekMoE 16B with 2 shared
and 64 routed experts, 6 of them active; MoonEP article, "basic usage":
S=4096, H=7168, K=8, E=256, 8 ranks, token_padding=128, and its maxvio
imbalance measure).
"""
from __future__ import annotations

import dataclasses
from typing import Optional

import numpy as np
import torch

BASE_SEED = 20261203

PAD_NONE = 0
PAD_MULTIPLE = 1
PAD_CAPACITY = 2

# tensor tags for SeedSequence
_TAG_HIDDEN = 1
_TAG_ROUTING = 2
_TAG_WEIGHTS = 3
_TAG_SHARED_A = 4
_TAG_SHARED_B = 5
_TAG_EXPERT_OUT = 6
_TAG_STAMPED = 7


@dataclasses.dataclass(frozen=True)
class WorkloadConfig:
    name: str
    S: int            # tokens
    H: int            # hidden size (bf16 channels)
    E: int            # routed experts
    K: int            # experts per token
    R: int            # simulated EP ranks (E % R == 0)
    fp8: bool = False
    pad_mode: int = PAD_NONE
    pad_rows: int = 0
    routing: str = "uniform"      # uniform | group_limited | zipf
    n_groups: int = 1             # group_limited: expert groups
    topk_groups: int = 1          # group_limited: groups kept per token
    target_maxvio: float = 0.0    # zipf: max load / mean load - 1
    shared: bool = False          # combine adds a shared-expert output
    seed_index: int = 0

    def describe(self) -> dict:
        d = dataclasses.asdict(self)
        d.pop("seed_index")
        return d


CONFIGS = {
    "tiny": WorkloadConfig("tiny", S=256, H=512, E=16, K=2, R=4, seed_index=0),
    "prefill": WorkloadConfig("prefill", S=4096, H=7168, E=256, K=8, R=8, fp8=True,
                              routing="group_limited", n_groups=8, topk_groups=4,
                              seed_index=1),
    "decode": WorkloadConfig("decode", S=128, H=7168, E=256, K=8, R=8, fp8=True,
                             pad_mode=PAD_CAPACITY, pad_rows=128, seed_index=2),
    "skew": WorkloadConfig("skew", S=4096, H=7168, E=256, K=8, R=8,
                           pad_mode=PAD_MULTIPLE, pad_rows=128, routing="zipf",
                           target_maxvio=20.0, seed_index=3),
    "dsmoe16b": WorkloadConfig("dsmoe16b", S=16384, H=2048, E=64, K=6, R=8,
                               shared=True, seed_index=4),
}


def _rng(seed: int, tag: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(np.random.SeedSequence([seed, tag])))


def _f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)


def normal_bf16_bits(rng: np.random.Generator, shape) -> np.ndarray:
    """N(0,1) drawn in fp32, stored as bf16 bit patterns (uint16)."""
    return _f32_to_bf16_bits(rng.standard_normal(size=shape, dtype=np.float32))


def softmax_weights(logits: np.ndarray) -> np.ndarray:
    """Route weights: softmax over the K picks of each token (fp64 math, fp32 out)."""
    z = logits.astype(np.float64)
    z = z - z.max(axis=1, keepdims=True)
    ez = np.exp(z)
    return (ez / ez.sum(axis=1, keepdims=True)).astype(np.float32)


def uniform_distinct_routing(rng: np.random.Generator, S: int, E: int, K: int) -> np.ndarray:
    """K distinct experts per token, every K-subset equally likely, in random order."""
    if K > E:
        raise ValueError("K distinct experts need K <= E")
    keys = rng.random((S, E))
    return np.argsort(keys, axis=1, kind="stable")[:, :K].astype(np.int32)


def group_limited_routing(rng: np.random.Generator, S: int, E: int, K: int,
                          n_groups: int, topk_groups: int):
    """Group-limited gating: keep the ``topk_groups`` groups with the highest
    max score, then the top-K scores among their experts.

    Groups are contiguous id ranges of E/n_groups experts.  Ties go to the lower
    index; the K picks are returned in descending score order, with their
    softmax weights.
    """
    if E % n_groups:
        raise ValueError("E must split into equal groups")
    gsize = E // n_groups
    z = rng.standard_normal(size=(S, E), dtype=np.float32)
    gmax = z.reshape(S, n_groups, gsize).max(axis=2)
    top_groups = np.argsort(-gmax, axis=1, kind="stable")[:, :topk_groups]
    allowed = np.zeros((S, n_groups), dtype=bool)
    np.put_along_axis(allowed, top_groups, True, axis=1)
    allowed_e = np.repeat(allowed, gsize, axis=1)
    zm = np.where(allowed_e, z, -np.inf)
    idx = np.argsort(-zm, axis=1, kind="stable")[:, :K]
    w = softmax_weights(np.take_along_axis(z, idx, axis=1))
    return idx.astype(np.int32), w


def maxvio(topk_idx: np.ndarray, E: int) -> float:
    """Max expert load over the mean load, minus one (MoonEP's imbalance measure)."""
    counts = np.bincount(topk_idx.reshape(-1), minlength=E)
    return float(counts.max() / (topk_idx.size / E) - 1.0)


def zipf_routing(rng: np.random.Generator, S: int, E: int, K: int,
                 target_maxvio: float, tol: float = 0.5):
    """Skewed routing: K distinct experts per token sampled without replacement
    from p_e ~ (e+1)^-s (Gumbel-top-K), with s bisected until maxvio is within
    ``tol`` of the target.  Expert 0 is the hottest.  Returns (idx, s)."""
    u = rng.random((S, E))
    with np.errstate(divide="ignore"):
        g = -np.log(-np.log(u))
    logr = np.log(np.arange(1, E + 1, dtype=np.float64))

    def pick(s: float) -> np.ndarray:
        keys = g - s * logr
        idx = np.argsort(-keys, axis=1, kind="stable")[:, :K]
        return idx.astype(np.int32)

    lo, hi = 0.0, 8.0
    for _ in range(80):
        mid = 0.5 * (lo + hi)
        idx = pick(mid)
        mv = maxvio(idx, E)
        if abs(mv - target_maxvio) <= tol:
            return idx, mid
        if mv < target_maxvio:
            lo = mid
        else:
            hi = mid
    raise RuntimeError("could not reach the requested maxvio")


@dataclasses.dataclass
class Workload:
    cfg: WorkloadConfig
    seed: int
    hidden: np.ndarray            # uint16 [S, H] bf16 bits
    topk_idx: np.ndarray          # int32  [S, K]
    topk_w: np.ndarray            # float32 [S, K]
    shared: Optional[np.ndarray]  # uint16 [S, H] bf16 bits or None
    zipf_s: Optional[float] = None


def make_workload(cfg: WorkloadConfig, seed: Optional[int] = None,
                  with_hidden: bool = True) -> Workload:
    """Draw one batch of inputs for ``cfg``.  ``seed`` defaults to
    BASE_SEED + cfg.seed_index."""
    if seed is None:
        seed = BASE_SEED + cfg.seed_index
    S, H, E, K = cfg.S, cfg.H, cfg.E, cfg.K
    hidden = normal_bf16_bits(_rng(seed, _TAG_HIDDEN), (S, H)) if with_hidden else None
    rrng = _rng(seed, _TAG_ROUTING)
    zipf_s = None
    if cfg.routing == "uniform":
        idx = uniform_distinct_routing(rrng, S, E, K)
        w = softmax_weights(_rng(seed, _TAG_WEIGHTS).standard_normal((S, K), dtype=np.float32))
    elif cfg.routing == "group_limited":
        idx, w = group_limited_routing(rrng, S, E, K, cfg.n_groups, cfg.topk_groups)
    elif cfg.routing == "zipf":
        idx, zipf_s = zipf_routing(rrng, S, E, K, cfg.target_maxvio)
        w = softmax_weights(_rng(seed, _TAG_WEIGHTS).standard_normal((S, K), dtype=np.float32))
    else:
        raise ValueError(f"unknown routing {cfg.routing!r}")
    shared = None
    if cfg.shared:
        a = torch.from_numpy(normal_bf16_bits(_rng(seed, _TAG_SHARED_A), (S, H)).view(np.int16))
        b = torch.from_numpy(normal_bf16_bits(_rng(seed, _TAG_SHARED_B), (S, H)).view(np.int16))
        # output of the two shared experts, summed by the model and stored as bf16
        s = a.view(torch.bfloat16).float() + b.view(torch.bfloat16).float()
        shared = s.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    return Workload(cfg=cfg, seed=seed, hidden=hidden, topk_idx=np.ascontiguousarray(idx),
                    topk_w=np.ascontiguousarray(w), shared=shared, zipf_s=zipf_s)


def random_expert_out_bits(seed: int, rows: int, H: int,
                           row_mask: Optional[np.ndarray] = None,
                           poison: int = 0x7FC1) -> np.ndarray:
    """Stand-in expert outputs [rows, H] bf16 ~ N(0,1).  Rows outside
    ``row_mask`` hold a NaN pattern, so reading one shows up in any result."""
    out = np.full((rows, H), poison, dtype=np.uint16)
    rng = _rng(seed, _TAG_EXPERT_OUT)
    if row_mask is None:
        out[:] = normal_bf16_bits(rng, (rows, H))
    else:
        sel = np.nonzero(row_mask)[0]
        out[sel] = normal_bf16_bits(rng, (sel.size, H))
    return out


def stamped_rows_bf16_bits(seed: int, S: int, H: int, base_rows: int = 1024) -> np.ndarray:
    """Token rows [S, H] bf16 bits for batches too large to draw row by row:
    row t is row t % base_rows of an N(0,1) table, and in every 512-channel
    chunk c the first four channels hold the small integers t & 255,
    (t >> 8) & 255, t >> 16 and c & 255 (exact in bf16), so a row or a chunk
    that lands in another token's or chunk's place cannot match.  H must be a
    multiple of 8 and S < 2**24."""
    if H % 8 or not 0 <= S < (1 << 24):
        raise ValueError("H must be a multiple of 8 and S < 2**24")
    base = normal_bf16_bits(_rng(seed, _TAG_STAMPED), (base_rows, H))
    out = np.empty((S, H), dtype=np.uint16)
    for i in range(0, S, base_rows):
        n = min(base_rows, S - i)
        out[i:i + n] = base[:n]
    small = (np.arange(256, dtype=np.float32).view(np.uint32) >> 16).astype(np.uint16)
    t = np.arange(S)
    for c, col in enumerate(range(0, H, 512)):
        out[:, col] = small[t & 255]
        out[:, col + 1] = small[(t >> 8) & 255]
        out[:, col + 2] = small[t >> 16]
        out[:, col + 3] = small[c & 255]
    return out
