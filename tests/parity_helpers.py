"""Shared helpers for the GPU parity tests: move numpy inputs to the device,
run the HIP path through the C ABI, and compare with the CPU oracle."""
from __future__ import annotations

import numpy as np
import torch

POISON_BF16 = 0x7FA5   # a NaN pattern: if it shows up in a result, a padding row was read
POISON_U8 = 0xA5


def dev_bf16(bits: np.ndarray, dev) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(dev).view(torch.bfloat16)


def host_bits(t: torch.Tensor) -> np.ndarray:
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def ordered(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns -> integers ordered like the values (+0 and -0 are 1 apart)."""
    b = bits.astype(np.int64)
    return np.where(b & 0x8000, 0xFFFF - b, b + 0x8000)


def bf16_value(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def assert_combine_matches(got: np.ndarray, ref: np.ndarray, what: str = "combine"):
    """The combine bar: every element within 1 bf16 ulp of the oracle (ordered
    bit distance <= 1) and max |got - ref| <= 1e-2 * max |ref|.  Returns the
    number of elements that are not bit-identical."""
    assert got.shape == ref.shape
    d = np.abs(ordered(got) - ordered(ref))
    worst = int(d.max()) if d.size else 0
    assert worst <= 1, f"{what}: {int((d > 1).sum())} elements differ by more than 1 ulp (max {worst})"
    if d.size:
        gv, rv = bf16_value(got), bf16_value(ref)
        assert np.all(np.isfinite(gv)), f"{what}: non-finite output"
        assert np.max(np.abs(gv - rv)) <= 1e-2 * np.max(np.abs(rv)) + 0.0
    return int((d != 0).sum())


def compare_layout(lay, ref, what: str = "layout"):
    for name, want in ref.as_dict().items():
        got = getattr(lay, name).cpu().numpy().reshape(want.shape)
        if not np.array_equal(got, want):
            bad = np.nonzero(got.reshape(-1) != want.reshape(-1))[0]
            raise AssertionError(f"{what}.{name}: {bad.size} mismatches, first at {bad[:5].tolist()}: "
                                 f"got {got.reshape(-1)[bad[:5]].tolist()} want {want.reshape(-1)[bad[:5]].tolist()}")
