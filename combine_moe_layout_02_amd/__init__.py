"""MI355X-native MoE expert-parallel layout, dispatch and combine.

Thin ctypes binding over libmoe_ep.so (declared in include/moe_ep.h).  The
Python functions carry the C names and only marshal arguments: torch tensors
supply device memory and the current HIP stream, every step of the path runs
in the library's HIP kernels.  Importing this package fails loudly when the
library has not been built; there is no CPU fallback.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmoe_ep.so")

MOE_OK, MOE_ERR_NULL, MOE_ERR_SHAPE, MOE_ERR_ALIGN, MOE_ERR_WORKSPACE, MOE_ERR_HIP = range(6)
MOE_PAD_NONE, MOE_PAD_MULTIPLE, MOE_PAD_CAPACITY = 0, 1, 2
MOE_FLAG_BAD_EXPERT, MOE_FLAG_CAPACITY, MOE_FLAG_UNBALANCED = 1, 2, 4

EXPORTED = ("moe_max_recv_rows", "moe_layout_workspace_bytes", "moe_layout", "moe_dispatch",
            "moe_layout_dispatch", "moe_combine", "moe_layout_balanced_workspace_bytes", "moe_layout_balanced",
            "moe_zero_padding", "moe_stream_create_cu_limited", "moe_stream_create_cu_range", "moe_stream_destroy",
            "moe_status_str", "moe_layout_noalloc")


class MoeError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {_lib.moe_status_str(status).decode()}")


class moe_layout_desc(ctypes.Structure):
    _fields_ = [("S", ctypes.c_int32), ("K", ctypes.c_int32), ("E", ctypes.c_int32),
                ("R", ctypes.c_int32), ("pad_mode", ctypes.c_int32), ("pad_rows", ctypes.c_int32)]


class moe_layout_bufs(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("tokens_per_expert", "tokens_per_rank", "expert_offset",
                                               "rank_offset", "pos", "src", "status")]


class moe_balance_bufs(ctypes.Structure):
    _fields_ = [("seg_offset", ctypes.c_void_p), ("slot_expert", ctypes.c_void_p)]


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; "
                          "g.build()'` (hipcc, gfx950); there is no fallback path")
    L = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    D = ctypes.POINTER(moe_layout_desc)
    B = ctypes.POINTER(moe_layout_bufs)
    L.moe_max_recv_rows.argtypes = [D]
    L.moe_max_recv_rows.restype = ctypes.c_int64
    L.moe_layout_workspace_bytes.argtypes = [D]
    L.moe_layout_workspace_bytes.restype = ctypes.c_size_t
    L.moe_layout.argtypes = [D, P, B, P, ctypes.c_size_t, P]
    L.moe_layout.restype = ctypes.c_int
    L.moe_dispatch.argtypes = [D, B, P, ctypes.c_int32, P, P, ctypes.c_int32, P, P, P, P]
    L.moe_dispatch.restype = ctypes.c_int
    L.moe_layout_dispatch.argtypes = [D, P, B, P, ctypes.c_size_t, P, ctypes.c_int32, P, ctypes.c_int32,
                                      P, P, P, P]
    L.moe_layout_dispatch.restype = ctypes.c_int
    L.moe_combine.argtypes = [D, B, P, ctypes.c_int32, P, P, P, P]
    L.moe_combine.restype = ctypes.c_int
    L.moe_zero_padding.argtypes = [D, B, ctypes.c_int32, ctypes.c_int32, P, P, P]
    L.moe_zero_padding.restype = ctypes.c_int
    L.moe_layout_balanced_workspace_bytes.argtypes = [D, ctypes.c_int32]
    L.moe_layout_balanced_workspace_bytes.restype = ctypes.c_size_t
    L.moe_layout_balanced.argtypes = [D, ctypes.c_int32, P, B, ctypes.POINTER(moe_balance_bufs), P,
                                      ctypes.c_size_t, P]
    L.moe_layout_balanced.restype = ctypes.c_int
    L.moe_stream_create_cu_limited.argtypes = [ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    L.moe_stream_create_cu_limited.restype = ctypes.c_int
    L.moe_stream_create_cu_range.argtypes = [ctypes.c_int32, ctypes.c_int32, ctypes.POINTER(ctypes.c_void_p)]
    L.moe_stream_create_cu_range.restype = ctypes.c_int
    L.moe_stream_destroy.argtypes = [P]
    L.moe_stream_destroy.restype = ctypes.c_int
    L.moe_status_str.argtypes = [ctypes.c_int32]
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_layout_noalloc.argtypes = [D, P, B, P]
    L.moe_layout_noalloc.restype = ctypes.c_int
    return L


_lib = _load()


def lib() -> ctypes.CDLL:
    return _lib


# ---------------------------------------------------------------------------
# descriptors
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class LayoutDesc:
    S: int
    K: int
    E: int
    R: int
    pad_mode: int = MOE_PAD_NONE
    pad_rows: int = 0

    def c(self) -> moe_layout_desc:
        return moe_layout_desc(self.S, self.K, self.E, self.R, self.pad_mode, self.pad_rows)


@dataclasses.dataclass
class Layout:
    """Device tensors of one batch's layout (outputs of moe_layout)."""
    tokens_per_expert: torch.Tensor   # [E] int32
    tokens_per_rank: torch.Tensor     # [R] int32
    expert_offset: torch.Tensor       # [E+1] int32
    rank_offset: torch.Tensor         # [R+1] int32
    pos: torch.Tensor                 # [S,K] int32
    src: torch.Tensor                 # [max_recv] int32
    status: torch.Tensor              # [1] int32
    workspace: Optional[torch.Tensor] = None

    def c(self) -> moe_layout_bufs:
        return moe_layout_bufs(*(t.data_ptr() for t in (
            self.tokens_per_expert, self.tokens_per_rank, self.expert_offset, self.rank_offset,
            self.pos, self.src, self.status)))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else t.data_ptr()   # argtypes make it a void*


# torch's raw current-stream query: measured ~0.1 us per call against ~2 us
# for torch.cuda.current_stream(), which builds a Stream object.  A
# decode-sized call costs only a few microseconds on the GPU, so the host side
# of every call counts.
_raw_current_stream = getattr(torch._C, "_cuda_getCurrentRawStream", None)


def _stream(stream, device) -> int:
    """Raw hipStream_t of `stream`, or of the current stream of `device`."""
    if stream is not None:
        return stream.cuda_stream
    if _raw_current_stream is not None:
        return _raw_current_stream(device.index)
    return torch.cuda.current_stream(device).cuda_stream


def _check(t: Optional[torch.Tensor], name: str, dtype, shape=None, device=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name}: dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: shape {tuple(t.shape)}, expected {tuple(shape)}")
    if device is not None and t.device != device:
        raise ValueError(f"{name} is on {t.device}, expected {device}")


# ---------------------------------------------------------------------------
# the C calls
# ---------------------------------------------------------------------------

def moe_max_recv_rows(desc: LayoutDesc) -> int:
    d = desc.c()
    return int(_lib.moe_max_recv_rows(ctypes.byref(d)))


def moe_layout_workspace_bytes(desc: LayoutDesc) -> int:
    d = desc.c()
    return int(_lib.moe_layout_workspace_bytes(ctypes.byref(d)))


def moe_status_str(status: int) -> str:
    return _lib.moe_status_str(int(status)).decode()


class PingPongBuffer:
    """Two Buffers of one shape used in turn: call i works in buffer i % 2, so
    the results of call i stay valid while call i + 1 runs -- the double
    buffer of DeepEP's low-latency kernels (DeepEP analysis, code notes).
    ``next()`` returns the buffer for the next call; arguments as Buffer."""

    def __init__(self, *args, **kwargs):
        self.buffers = (Buffer(*args, **kwargs), Buffer(*args, **kwargs))
        self._i = 0

    def next(self) -> "Buffer":
        b = self.buffers[self._i]
        self._i ^= 1
        return b


class CULimitedStream:
    """A HIP stream whose kernels run only on CUs [first_cu, first_cu +
    num_cus) (moe_stream_create_cu_range; first_cu = 0 is
    moe_stream_create_cu_limited), usable as a torch stream."""

    def __init__(self, num_cus: int, device="cuda", first_cu: int = 0):
        handle = ctypes.c_void_p()
        rc = _lib.moe_stream_create_cu_range(int(first_cu), int(num_cus), ctypes.byref(handle))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_stream_create_cu_range")
        self.num_cus = num_cus
        self.handle = handle.value
        self.stream = torch.cuda.ExternalStream(self.handle, device=torch.device(device))

    def close(self):
        if self.handle:
            torch.cuda.synchronize()
            _lib.moe_stream_destroy(ctypes.c_void_p(self.handle))
            self.handle = None

    def __enter__(self):
        return self

    def __exit__(self, *exc):
        self.close()


def alloc_layout(desc: LayoutDesc, device) -> Layout:
    """Device buffers for moe_layout's outputs and its workspace (torch memory)."""
    rows = moe_max_recv_rows(desc)
    if rows < 0:
        raise MoeError(MOE_ERR_SHAPE, "alloc_layout")
    i32 = dict(dtype=torch.int32, device=device)
    ws = moe_layout_workspace_bytes(desc)
    return Layout(
        tokens_per_expert=torch.empty(desc.E, **i32), tokens_per_rank=torch.empty(desc.R, **i32),
        expert_offset=torch.empty(desc.E + 1, **i32), rank_offset=torch.empty(desc.R + 1, **i32),
        pos=torch.empty((desc.S, desc.K), **i32), src=torch.empty(rows, **i32),
        status=torch.empty(1, **i32),
        workspace=torch.empty(ws, dtype=torch.uint8, device=device) if ws else None)


def moe_layout(desc: LayoutDesc, topk_idx: torch.Tensor, layout: Optional[Layout] = None,
               stream=None) -> Layout:
    dev = topk_idx.device
    _check(topk_idx, "topk_idx", torch.int32, (desc.S, desc.K))
    if layout is None:
        layout = alloc_layout(desc, dev)
    ws = layout.workspace
    d, b = desc.c(), layout.c()
    rc = _lib.moe_layout(ctypes.byref(d), _ptr(topk_idx), ctypes.byref(b), _ptr(ws),
                         0 if ws is None else ws.numel(), _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layout")
    return layout


def moe_layout_noalloc(desc: LayoutDesc, topk_idx: torch.Tensor, layout: Layout, stream=None) -> Layout:
    """moe_layout with the library's own per-GPU scratch instead of a
    workspace: the C call allocates nothing (the output tensors of `layout`
    are the caller's; its workspace, if any, is not used)."""
    dev = topk_idx.device
    _check(topk_idx, "topk_idx", torch.int32, (desc.S, desc.K))
    d, b = desc.c(), layout.c()
    rc = _lib.moe_layout_noalloc(ctypes.byref(d), _ptr(topk_idx), ctypes.byref(b), _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layout_noalloc")
    return layout


def moe_dispatch(desc: LayoutDesc, layout: Layout, hidden: torch.Tensor, topk_idx=None, topk_w=None,
                 fp8: bool = False, recv=None, recv_scales=None, recv_w=None, stream=None):
    """Returns (recv, recv_scales or None, recv_w or None).  recv is bf16
    [max_recv,H], or uint8 E4M3FN codes [max_recv,H] when fp8."""
    dev = hidden.device
    S, H = hidden.shape
    rows = moe_max_recv_rows(desc)
    _check(hidden, "hidden", torch.bfloat16, (desc.S, H))
    _check(topk_w, "topk_w", torch.float32, (desc.S, desc.K))
    if recv is None:
        recv = torch.empty((rows, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
    if recv_w is None and topk_w is not None:
        recv_w = torch.empty(rows, dtype=torch.float32, device=dev)
    _check(recv, "recv", (torch.uint8, torch.float8_e4m3fn) if fp8 else torch.bfloat16)
    if recv.shape[0] < rows or recv.shape[-1] != H:
        raise ValueError("recv must hold moe_max_recv_rows rows of H channels")
    if fp8:
        _check(recv_scales, "recv_scales", torch.float32)
        if recv_scales.shape[0] < rows or recv_scales.shape[-1] != H // 128:
            raise ValueError("recv_scales must be [max_recv, H/128]")
    _check(recv_w, "recv_w", torch.float32)
    d, b = desc.c(), layout.c()
    rc = _lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), _ptr(hidden), H, _ptr(topk_idx), _ptr(topk_w),
                           1 if fp8 else 0, _ptr(recv), _ptr(recv_scales if fp8 else None), _ptr(recv_w),
                           _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_dispatch")
    return recv, (recv_scales if fp8 else None), recv_w


def moe_layout_balanced_workspace_bytes(desc: LayoutDesc, slots_per_rank: int) -> int:
    d = desc.c()
    return int(_lib.moe_layout_balanced_workspace_bytes(ctypes.byref(d), int(slots_per_rank)))


@dataclasses.dataclass
class Balance:
    """Device outputs of moe_layout_balanced beyond the layout."""
    seg_offset: torch.Tensor    # [R*(E/R+B)+1] int32
    slot_expert: torch.Tensor   # [R*B] int32
    workspace: Optional[torch.Tensor]   # scratch (uint8), None when none is needed

    def c(self) -> moe_balance_bufs:
        return moe_balance_bufs(self.seg_offset.data_ptr(), self.slot_expert.data_ptr())


def alloc_balance(desc: LayoutDesc, slots_per_rank: int, device) -> Balance:
    epr = desc.E // desc.R
    ws = moe_layout_balanced_workspace_bytes(desc, slots_per_rank)
    return Balance(torch.empty(desc.R * (epr + slots_per_rank) + 1, dtype=torch.int32, device=device),
                   torch.empty(max(desc.R * slots_per_rank, 1), dtype=torch.int32, device=device),
                   torch.empty(ws, dtype=torch.uint8, device=device) if ws else None)


def moe_layout_balanced(desc: LayoutDesc, slots_per_rank: int, topk_idx: torch.Tensor,
                        layout: Optional[Layout] = None, balance: Optional[Balance] = None, stream=None):
    """Balanced layout (equal rows per rank through redundant-expert slots).
    Returns (layout, balance)."""
    dev = topk_idx.device
    _check(topk_idx, "topk_idx", torch.int32, (desc.S, desc.K))
    if layout is None:
        layout = alloc_layout(desc, dev)
    if balance is None:
        balance = alloc_balance(desc, slots_per_rank, dev)
    d, b, bb = desc.c(), layout.c(), balance.c()
    rc = _lib.moe_layout_balanced(ctypes.byref(d), int(slots_per_rank), _ptr(topk_idx), ctypes.byref(b),
                                  ctypes.byref(bb), _ptr(balance.workspace),
                                  0 if balance.workspace is None else balance.workspace.numel(),
                                  _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layout_balanced")
    return layout, balance


def moe_layout_dispatch(desc: LayoutDesc, topk_idx: torch.Tensor, hidden: torch.Tensor, topk_w=None,
                        fp8: bool = False, layout: Optional[Layout] = None, recv=None, recv_scales=None,
                        recv_w=None, stream=None):
    """moe_layout + moe_dispatch in one call (one launch for S*K <= 4096 and S <= 512).
    Returns (layout, recv, recv_scales or None, recv_w or None)."""
    dev = hidden.device
    H = hidden.shape[1]
    rows = moe_max_recv_rows(desc)
    _check(topk_idx, "topk_idx", torch.int32, (desc.S, desc.K))
    _check(hidden, "hidden", torch.bfloat16, (desc.S, H))
    _check(topk_w, "topk_w", torch.float32, (desc.S, desc.K))
    if layout is None:
        layout = alloc_layout(desc, dev)
    if recv is None:
        recv = torch.empty((rows, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
    if fp8 and recv_scales is None:
        recv_scales = torch.empty((rows, H // 128), dtype=torch.float32, device=dev)
    if recv_w is None and topk_w is not None:
        recv_w = torch.empty(rows, dtype=torch.float32, device=dev)
    _check(recv, "recv", (torch.uint8, torch.float8_e4m3fn) if fp8 else torch.bfloat16)
    if recv.shape[0] < rows or recv.shape[-1] != H:
        raise ValueError("recv must hold moe_max_recv_rows rows of H channels")
    if fp8:
        _check(recv_scales, "recv_scales", torch.float32)
        if recv_scales.shape[0] < rows or recv_scales.shape[-1] != H // 128:
            raise ValueError("recv_scales must be [max_recv, H/128]")
    _check(recv_w, "recv_w", torch.float32)
    ws = layout.workspace
    d, b = desc.c(), layout.c()
    rc = _lib.moe_layout_dispatch(ctypes.byref(d), _ptr(topk_idx), ctypes.byref(b), _ptr(ws),
                                  0 if ws is None else ws.numel(), _ptr(hidden), H, _ptr(topk_w),
                                  1 if fp8 else 0, _ptr(recv), _ptr(recv_scales if fp8 else None), _ptr(recv_w),
                                  _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_layout_dispatch")
    return layout, recv, (recv_scales if fp8 else None), recv_w


def moe_combine(desc: LayoutDesc, layout: Layout, expert_out: torch.Tensor, w=None, shared_out=None,
                out=None, stream=None) -> torch.Tensor:
    dev = expert_out.device
    H = expert_out.shape[-1]
    _check(expert_out, "expert_out", torch.bfloat16)
    if expert_out.shape[0] < moe_max_recv_rows(desc):
        raise ValueError("expert_out must hold moe_max_recv_rows rows")
    _check(w, "w", torch.float32, (desc.S, desc.K))
    _check(shared_out, "shared_out", torch.bfloat16, (desc.S, H))
    if out is None:
        out = torch.empty((desc.S, H), dtype=torch.bfloat16, device=dev)
    _check(out, "out", torch.bfloat16, (desc.S, H))
    d, b = desc.c(), layout.c()
    rc = _lib.moe_combine(ctypes.byref(d), ctypes.byref(b), _ptr(expert_out), H, _ptr(w), _ptr(shared_out),
                          _ptr(out), _stream(stream, dev))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_combine")
    return out


def moe_zero_padding(desc: LayoutDesc, layout: Layout, recv: torch.Tensor, recv_scales=None, stream=None):
    """Zero every receive row that no entry maps to (and its FP8 scales).
    FP8 when recv holds E4M3 codes (uint8 or float8_e4m3fn), bf16 otherwise."""
    fp8 = recv.dtype in (torch.uint8, torch.float8_e4m3fn)
    H = recv.shape[-1]
    _check(recv, "recv", (torch.uint8, torch.float8_e4m3fn) if fp8 else torch.bfloat16)
    if recv.shape[0] < moe_max_recv_rows(desc):
        raise ValueError("recv must hold moe_max_recv_rows rows")
    if fp8:
        _check(recv_scales, "recv_scales", torch.float32, (recv.shape[0], H // 128))
    d, b = desc.c(), layout.c()
    rc = _lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), H, 1 if fp8 else 0, _ptr(recv),
                               _ptr(recv_scales) if fp8 else None, _stream(stream, recv.device))
    if rc != MOE_OK:
        raise MoeError(rc, "moe_zero_padding")


# ---------------------------------------------------------------------------
# Static-shape buffer: validate once, then bare C calls
# ---------------------------------------------------------------------------

class Buffer:
    """All device buffers of one batch shape, allocated once (static shapes, no
    host sync between layers), with prepared C calls.

    Mirrors the call shape of MoonEP's Buffer (MoonEP article, basic usage):
    ``dispatch(hidden, topk_w, topk_idx)`` returns the expert-grouped rows,
    their per-row weights and the per-expert offsets; ``combine(expert_out)``
    returns the token-order result.  Every call is asynchronous on the current
    stream (or the one given); outputs are views of the buffer's own tensors
    and are overwritten by the next call.

    With ``balance_slots=B`` the layout is the balanced one (moe_layout_balanced:
    every rank receives the same number of rows, the surplus of hot experts
    going to B replica slots per rank; MoonEP article, section 1); dispatch and
    combine are unchanged.  ``balance.slot_expert`` then tells which expert each
    slot must hold.
    """

    def __init__(self, S: int, H: int, K: int, E: int, R: int, fp8: bool = False,
                 pad_mode: int = MOE_PAD_NONE, pad_rows: int = 0, device="cuda",
                 balance_slots: Optional[int] = None):
        if balance_slots is not None and pad_mode != MOE_PAD_NONE:
            raise MoeError(MOE_ERR_SHAPE, "Buffer: the balanced layout has no padding")
        self.desc = LayoutDesc(S, K, E, R, pad_mode, pad_rows)
        self.rows = moe_max_recv_rows(self.desc)
        if self.rows < 0 or H < 8 or H % 8 or (fp8 and H % 128):
            raise MoeError(MOE_ERR_SHAPE, "Buffer")
        dev = torch.device(device)
        if dev.type == "cuda" and dev.index is None:
            dev = torch.device("cuda", torch.cuda.current_device())
        self.H, self.fp8, self.device = H, fp8, dev
        self.layout = alloc_layout(self.desc, dev)
        self.recv = torch.empty((self.rows, H), dtype=torch.uint8 if fp8 else torch.bfloat16, device=dev)
        self.recv_scales = torch.empty((self.rows, H // 128), dtype=torch.float32, device=dev) if fp8 else None
        self.recv_w = torch.empty(self.rows, dtype=torch.float32, device=dev)
        self.out = torch.empty((S, H), dtype=torch.bfloat16, device=dev)
        self._d = self.desc.c()
        self._b = self.layout.c()
        self._dp = ctypes.byref(self._d)
        self._bp = ctypes.byref(self._b)
        ws = self.layout.workspace
        self._ws = (_ptr(ws), 0 if ws is None else ws.numel())
        self._recv = _ptr(self.recv)
        self._scales = _ptr(self.recv_scales)
        self._recv_w = _ptr(self.recv_w)
        self._out = _ptr(self.out)
        self.balance, self.slots = None, balance_slots
        if balance_slots is not None:
            self.balance = alloc_balance(self.desc, balance_slots, dev)
            self._bal = self.balance.c()
            self._balp = ctypes.byref(self._bal)
            bws = self.balance.workspace
            self._bws = (_ptr(bws), 0 if bws is None else bws.numel())

    def _inputs(self, hidden, topk_idx, topk_w):
        S, K = self.desc.S, self.desc.K
        _check(topk_idx, "topk_idx", torch.int32, (S, K), self.device)
        _check(hidden, "hidden", torch.bfloat16, (S, self.H), self.device)
        _check(topk_w, "topk_w", torch.float32, (S, K), self.device)

    def layout_call(self, topk_idx, stream=None, check=True):
        if check:
            _check(topk_idx, "topk_idx", torch.int32, (self.desc.S, self.desc.K), self.device)
        if self.balance is not None:
            rc = _lib.moe_layout_balanced(self._dp, self.slots, _ptr(topk_idx), self._bp, self._balp,
                                          self._bws[0], self._bws[1], _stream(stream, self.device))
            if rc != MOE_OK:
                raise MoeError(rc, "moe_layout_balanced")
            return
        rc = _lib.moe_layout(self._dp, _ptr(topk_idx), self._bp, self._ws[0], self._ws[1],
                             _stream(stream, self.device))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layout")

    def dispatch_call(self, hidden, topk_idx=None, topk_w=None, stream=None, check=True):
        if check:
            self._inputs(hidden, topk_idx, topk_w)
        rc = _lib.moe_dispatch(self._dp, self._bp, _ptr(hidden), self.H, _ptr(topk_idx), _ptr(topk_w),
                               1 if self.fp8 else 0, self._recv, self._scales,
                               self._recv_w if topk_w is not None else None, _stream(stream, self.device))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_dispatch")

    def layout_dispatch_call(self, hidden, topk_idx, topk_w=None, stream=None, check=True):
        """moe_layout_dispatch: one launch for decode-sized batches (with a
        balanced layout: the balanced layout, then moe_dispatch)."""
        if check:
            self._inputs(hidden, topk_idx, topk_w)
        if self.balance is not None:
            self.layout_call(topk_idx, stream, check=False)
            self.dispatch_call(hidden, topk_idx, topk_w, stream, check=False)
            return
        rc = _lib.moe_layout_dispatch(self._dp, _ptr(topk_idx), self._bp, self._ws[0], self._ws[1], _ptr(hidden),
                                      self.H, _ptr(topk_w), 1 if self.fp8 else 0, self._recv, self._scales,
                                      self._recv_w if topk_w is not None else None, _stream(stream, self.device))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_layout_dispatch")

    def combine_call(self, expert_out, w=None, shared_out=None, stream=None, check=True):
        if check:
            _check(expert_out, "expert_out", torch.bfloat16, (self.rows, self.H), self.device)
            _check(w, "w", torch.float32, (self.desc.S, self.desc.K), self.device)
            _check(shared_out, "shared_out", torch.bfloat16, (self.desc.S, self.H), self.device)
        rc = _lib.moe_combine(self._dp, self._bp, _ptr(expert_out), self.H, _ptr(w), _ptr(shared_out),
                              self._out, _stream(stream, self.device))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_combine")

    def zero_padding_call(self, stream=None):
        """moe_zero_padding on this buffer's receive rows (after a dispatch)."""
        rc = _lib.moe_zero_padding(self._dp, self._bp, self.H, 1 if self.fp8 else 0, self._recv, self._scales,
                                   _stream(stream, self.device))
        if rc != MOE_OK:
            raise MoeError(rc, "moe_zero_padding")

    def dispatch(self, hidden, topk_w, topk_idx, stream=None):
        """Layout + dispatch.  Returns (recv, recv_w, expert_offset, recv_scales)."""
        self.layout_dispatch_call(hidden, topk_idx, topk_w, stream)
        return self.recv, self.recv_w, self.layout.expert_offset, self.recv_scales

    def combine(self, expert_out, w=None, shared_out=None, stream=None):
        """Route-weighted gather back to token order.  Returns out [S,H] bf16."""
        self.combine_call(expert_out, w, shared_out, stream)
        return self.out
