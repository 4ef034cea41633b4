"""CPU oracle for MoE expert-parallel layout, dispatch and combine (ctypes front end).

TEST INFRASTRUCTURE ONLY.  The oracle is a plain, single-threaded C++ library
(``moe_oracle.cpp``, the plain C subset of C++) that shares no code with the
GPU library.  Only the test
suite, the smoke check and the benchmark's CPU-baseline leg may import this
package; the GPU path never calls it and never falls back to it.

All arrays are numpy: bf16 values travel as uint16 bit patterns, FP8 codes as
uint8.  Every function here only marshals arguments; the arithmetic is in C.
"""
from __future__ import annotations

import ctypes
import os
import subprocess
from typing import Optional

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(_HERE, "moe_oracle.cpp")
LIB = os.path.join(_HERE, "libmoe_oracle.so")

PAD_NONE, PAD_MULTIPLE, PAD_CAPACITY = 0, 1, 2
FLAG_BAD_EXPERT, FLAG_CAPACITY, FLAG_UNBALANCED = 1, 2, 4
OK, ERR_NULL, ERR_SHAPE = 0, 1, 2


def build() -> str:
    """Compile the oracle with g++ (IEEE fp32, no contraction)."""
    tmp = LIB + ".tmp"
    subprocess.run(["g++", "-O2", "-std=c++17", "-ffp-contract=off", "-fno-fast-math",
                    "-Wall", "-Wextra", "-shared", "-fPIC", "-o", tmp, SRC, "-lm"],
                   check=True)
    os.replace(tmp, LIB)
    return LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(LIB):
            raise FileNotFoundError(f"{LIB} is not built; run __graft_entry__.build()")
        L = ctypes.CDLL(LIB)
        P = ctypes.c_void_p
        i32, i64 = ctypes.c_int32, ctypes.c_int64
        L.oracle_f32_from_bf16.argtypes = [ctypes.c_uint16]
        L.oracle_f32_from_bf16.restype = ctypes.c_float
        L.oracle_bf16_from_f32.argtypes = [ctypes.c_float]
        L.oracle_bf16_from_f32.restype = ctypes.c_uint16
        L.oracle_f32_from_e4m3.argtypes = [ctypes.c_uint8]
        L.oracle_f32_from_e4m3.restype = ctypes.c_float
        L.oracle_e4m3_from_f32.argtypes = [ctypes.c_float]
        L.oracle_e4m3_from_f32.restype = ctypes.c_uint8
        L.oracle_max_recv_rows.argtypes = [i32] * 6
        L.oracle_max_recv_rows.restype = i64
        L.oracle_layout.argtypes = [P] + [i32] * 6 + [P] * 7
        L.oracle_layout.restype = i32
        L.oracle_dispatch_bf16.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.oracle_dispatch_bf16.restype = i32
        L.oracle_quantize_row_fp8.argtypes = [P, i32, P, P]
        L.oracle_quantize_row_fp8.restype = i32
        L.oracle_dispatch_fp8.argtypes = [P, i32, i32, i32, P, P, P, P, P]
        L.oracle_dispatch_fp8.restype = i32
        L.oracle_combine.argtypes = [P, i32, i32, i32, P, P, P, P]
        L.oracle_combine.restype = i32
        L.oracle_layout_balanced.argtypes = [P] + [i32] * 5 + [P] * 9
        L.oracle_layout_balanced.restype = i32
        L.oracle_bf16_from_f32_n.argtypes = [P, i64, P]
        L.oracle_bf16_from_f32_n.restype = None
        L.oracle_e4m3_from_f32_n.argtypes = [P, i64, P]
        L.oracle_e4m3_from_f32_n.restype = None
        L.oracle_dequant_identity.argtypes = [P, P, i64, i32, P]
        L.oracle_zero_padding.argtypes = [P, i64, i64, P, P, i32]
        L.oracle_zero_padding.restype = None
        L.oracle_dequant_identity.restype = None
        _lib = L
    return _lib


def _p(a: Optional[np.ndarray]):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _c(a, dtype):
    a = np.ascontiguousarray(a)
    if a.dtype != dtype:
        raise TypeError(f"expected {dtype}, got {a.dtype}")
    return a


# ---- number formats (scalar) ----------------------------------------------

def f32_from_bf16(h: int) -> float:
    return lib().oracle_f32_from_bf16(int(h))


def bf16_from_f32(v: float) -> int:
    return int(lib().oracle_bf16_from_f32(float(v)))


def f32_from_e4m3(c: int) -> float:
    return lib().oracle_f32_from_e4m3(int(c))


def e4m3_from_f32(v: float) -> int:
    return int(lib().oracle_e4m3_from_f32(float(v)))


def e4m3_from_f32_array(v: np.ndarray) -> np.ndarray:
    flat = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    out = np.zeros(flat.size, np.uint8)
    lib().oracle_e4m3_from_f32_n(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(v))


def bf16_from_f32_array(v: np.ndarray) -> np.ndarray:
    flat = np.ascontiguousarray(v, dtype=np.float32).reshape(-1)
    out = np.zeros(flat.size, np.uint16)
    lib().oracle_bf16_from_f32_n(_p(flat), flat.size, _p(out))
    return out.reshape(np.shape(v))


# ---- layout -----------------------------------------------------------------

def max_recv_rows(S, K, E, R, pad_mode=PAD_NONE, pad_rows=0) -> int:
    return int(lib().oracle_max_recv_rows(S, K, E, R, pad_mode, pad_rows))


class Layout:
    def __init__(self, tokens_per_expert, tokens_per_rank, expert_offset, rank_offset, pos, src, status):
        self.tokens_per_expert = tokens_per_expert
        self.tokens_per_rank = tokens_per_rank
        self.expert_offset = expert_offset
        self.rank_offset = rank_offset
        self.pos = pos
        self.src = src
        self.status = status

    def as_dict(self):
        return dict(tokens_per_expert=self.tokens_per_expert, tokens_per_rank=self.tokens_per_rank,
                    expert_offset=self.expert_offset, rank_offset=self.rank_offset,
                    pos=self.pos, src=self.src, status=self.status)


def layout(topk_idx: np.ndarray, E: int, R: int, pad_mode: int = PAD_NONE, pad_rows: int = 0) -> Layout:
    idx = _c(topk_idx, np.int32)
    S, K = idx.shape
    mr = max_recv_rows(S, K, E, R, pad_mode, pad_rows)
    if mr < 0:
        raise ValueError("bad layout shape")
    tpe = np.zeros(E, np.int32)
    tpr = np.zeros(R, np.int32)
    eoff = np.zeros(E + 1, np.int32)
    roff = np.zeros(R + 1, np.int32)
    pos = np.zeros((S, K), np.int32)
    src = np.zeros(mr, np.int32)
    status = np.zeros(1, np.int32)
    rc = lib().oracle_layout(_p(idx), S, K, E, R, pad_mode, pad_rows, _p(tpe), _p(tpr), _p(eoff),
                             _p(roff), _p(pos), _p(src), _p(status))
    if rc != OK:
        raise ValueError(f"oracle_layout failed with {rc}")
    return Layout(tpe, tpr, eoff, roff, pos, src, status)


class BalancedLayout(Layout):
    def __init__(self, seg_offset, slot_expert, **kw):
        super().__init__(**kw)
        self.seg_offset = seg_offset
        self.slot_expert = slot_expert

    def as_dict(self):
        d = super().as_dict()
        d.update(seg_offset=self.seg_offset, slot_expert=self.slot_expert)
        return d


def layout_balanced(topk_idx: np.ndarray, E: int, R: int, B: int) -> BalancedLayout:
    """Balanced layout with B redundant-expert slots per rank (see moe_oracle.cpp)."""
    idx = _c(topk_idx, np.int32)
    S, K = idx.shape
    if max_recv_rows(S, K, E, R) < 0 or not 0 <= B <= 64:
        raise ValueError("bad layout shape")
    epr = E // R
    out = dict(tokens_per_expert=np.zeros(E, np.int32), tokens_per_rank=np.zeros(R, np.int32),
               expert_offset=np.zeros(E + 1, np.int32), rank_offset=np.zeros(R + 1, np.int32),
               pos=np.zeros((S, K), np.int32), src=np.zeros(S * K, np.int32), status=np.zeros(1, np.int32))
    seg = np.zeros(R * (epr + B) + 1, np.int32)
    slot = np.zeros(R * B, np.int32)
    rc = lib().oracle_layout_balanced(_p(idx), S, K, E, R, B, _p(out["tokens_per_expert"]),
                                      _p(out["tokens_per_rank"]), _p(out["expert_offset"]),
                                      _p(out["rank_offset"]), _p(out["pos"]), _p(out["src"]), _p(seg),
                                      _p(slot), _p(out["status"]))
    if rc != OK:
        raise ValueError(f"oracle_layout_balanced failed with {rc}")
    return BalancedLayout(seg, slot, **out)


# ---- dispatch / combine -----------------------------------------------------

def dispatch_bf16(hidden: np.ndarray, pos: np.ndarray, max_recv: int, topk_w: Optional[np.ndarray] = None,
                  fill: int = 0):
    h = _c(hidden, np.uint16)
    p = _c(pos, np.int32)
    S, H = h.shape
    K = p.shape[1]
    recv = np.full((max_recv, H), fill, np.uint16)
    recv_w = np.zeros(max_recv, np.float32) if topk_w is not None else None
    w = _c(topk_w, np.float32) if topk_w is not None else None
    rc = lib().oracle_dispatch_bf16(_p(h), S, H, K, _p(p), _p(w), _p(recv), _p(recv_w))
    if rc != OK:
        raise ValueError(f"oracle_dispatch_bf16 failed with {rc}")
    return recv, recv_w


def quantize_row_fp8(row: np.ndarray):
    r = _c(row, np.uint16)
    H = r.shape[0]
    codes = np.zeros(H, np.uint8)
    scales = np.zeros(H // 128, np.float32)
    rc = lib().oracle_quantize_row_fp8(_p(r), H, _p(codes), _p(scales))
    if rc != OK:
        raise ValueError("bad row length")
    return codes, scales


def dispatch_fp8(hidden: np.ndarray, pos: np.ndarray, max_recv: int, topk_w: Optional[np.ndarray] = None,
                 fill: int = 0):
    h = _c(hidden, np.uint16)
    p = _c(pos, np.int32)
    S, H = h.shape
    K = p.shape[1]
    recv = np.full((max_recv, H), fill, np.uint8)
    scales = np.zeros((max_recv, H // 128), np.float32)
    recv_w = np.zeros(max_recv, np.float32) if topk_w is not None else None
    w = _c(topk_w, np.float32) if topk_w is not None else None
    rc = lib().oracle_dispatch_fp8(_p(h), S, H, K, _p(p), _p(w), _p(recv), _p(scales), _p(recv_w))
    if rc != OK:
        raise ValueError(f"oracle_dispatch_fp8 failed with {rc}")
    return recv, scales, recv_w


def combine(expert_out: np.ndarray, pos: np.ndarray, w: Optional[np.ndarray] = None,
            shared: Optional[np.ndarray] = None) -> np.ndarray:
    y = _c(expert_out, np.uint16)
    p = _c(pos, np.int32)
    S, K = p.shape
    H = y.shape[1]
    ww = _c(w, np.float32) if w is not None else None
    sh = _c(shared, np.uint16) if shared is not None else None
    out = np.zeros((S, H), np.uint16)
    rc = lib().oracle_combine(_p(y), S, H, K, _p(p), _p(ww), _p(sh), _p(out))
    if rc != OK:
        raise ValueError(f"oracle_combine failed with {rc}")
    return out


def zero_padding(src: np.ndarray, recv: np.ndarray, recv_scales=None):
    """Copies of recv (and recv_scales) with every row whose src is -1 zeroed."""
    srcs = _c(src, np.int32)
    out = np.array(recv, copy=True, order="C")
    rows = out.shape[0]
    row_bytes = out.reshape(rows, -1).view(np.uint8).shape[1]
    sc = None if recv_scales is None else np.array(recv_scales, dtype=np.float32, copy=True, order="C")
    lib().oracle_zero_padding(_p(srcs), rows, row_bytes, _p(out), None if sc is None else _p(sc),
                              0 if sc is None else sc.shape[1])
    return out, sc


def dequant_identity_expert(recv_codes: np.ndarray, recv_scales: np.ndarray) -> np.ndarray:
    """Stand-in 'identity expert' for FP8 rows: bf16(value(code) * scale) per
    element, with the oracle's own e4m3 decode and bf16 rounding."""
    codes = _c(recv_codes, np.uint8)
    scales = _c(recv_scales, np.float32)
    rows, H = codes.shape
    y = np.zeros((rows, H), np.uint16)
    lib().oracle_dequant_identity(_p(codes), _p(scales), rows, H, _p(y))
    return y
