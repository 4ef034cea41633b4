"""C-ABI checks that need no GPU: the library loads, exports every call the
header declares, sizes buffers like the oracle, and rejects bad arguments
synchronously (every case here returns before anything would be enqueued)."""
import ctypes
import os
import re

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


@pytest.fixture(scope="module")
def moe():
    from combine_moe_layout_02_amd.build import LIB
    if not os.path.exists(LIB):
        import __graft_entry__
        __graft_entry__.build()
    import combine_moe_layout_02_amd
    return combine_moe_layout_02_amd


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(moe_[a-z_0-9]+)\s*\(", text)))


def test_header_declarations_are_exported(moe):
    names = declared_functions()
    assert set(names) == set(moe.EXPORTED)
    lib = moe.lib()
    for n in names:
        assert getattr(lib, n) is not None


def test_max_recv_rows_and_workspace(moe):
    import oracle
    from workloads import CONFIGS
    for cfg in CONFIGS.values():
        d = moe.LayoutDesc(cfg.S, cfg.K, cfg.E, cfg.R, cfg.pad_mode, cfg.pad_rows)
        assert moe.moe_max_recv_rows(d) == oracle.max_recv_rows(cfg.S, cfg.K, cfg.E, cfg.R, cfg.pad_mode,
                                                                cfg.pad_rows)
    # the pages' shapes: decode buffer 256 experts x 128 rows; skew 32768 + 256*127
    assert moe.moe_max_recv_rows(moe.LayoutDesc(128, 8, 256, 8, moe.MOE_PAD_CAPACITY, 128)) == 32768
    assert moe.moe_max_recv_rows(moe.LayoutDesc(4096, 8, 256, 8, moe.MOE_PAD_MULTIPLE, 128)) == 65280
    assert moe.moe_layout_workspace_bytes(moe.LayoutDesc(128, 8, 256, 8)) == 0
    assert moe.moe_layout_workspace_bytes(moe.LayoutDesc(4096, 8, 256, 8)) == 0      # one launch, no scratch
    assert moe.moe_layout_workspace_bytes(moe.LayoutDesc(4097, 8, 256, 8)) >= 33 * 256 * 4
    for bad in [moe.LayoutDesc(8, 2, 8, 3), moe.LayoutDesc(8, 0, 8, 1), moe.LayoutDesc(8, 17, 32, 1),
                moe.LayoutDesc(8, 2, 1025, 1), moe.LayoutDesc(8, 2, 8, 2, moe.MOE_PAD_MULTIPLE, 0),
                moe.LayoutDesc(-1, 2, 8, 2), moe.LayoutDesc(8, 2, 8, 2, 7, 1),
                moe.LayoutDesc(1 << 28, 8, 8, 2), moe.LayoutDesc(8, 2, 1024, 1, moe.MOE_PAD_CAPACITY, 1 << 22)]:
        assert moe.moe_max_recv_rows(bad) == -1
        assert moe.moe_layout_workspace_bytes(bad) == 0


FAKE = 1 << 20  # a 16-byte aligned address that is never dereferenced


def _bufs(moe, misalign=None):
    fields = {n: FAKE + 4096 * i for i, (n, _) in enumerate(moe.moe_layout_bufs._fields_)}
    if misalign:
        fields[misalign] += 2
    return moe.moe_layout_bufs(**fields)


def test_layout_argument_errors(moe):
    lib = moe.lib()
    d = moe.LayoutDesc(64, 2, 8, 2).c()
    b = _bufs(moe)
    P = ctypes.c_void_p
    assert lib.moe_layout(None, P(FAKE), ctypes.byref(b), None, 0, None) == moe.MOE_ERR_NULL
    assert lib.moe_layout(ctypes.byref(d), P(FAKE), None, None, 0, None) == moe.MOE_ERR_NULL
    assert lib.moe_layout(ctypes.byref(d), None, ctypes.byref(b), None, 0, None) == moe.MOE_ERR_NULL
    bad = moe.LayoutDesc(64, 2, 8, 3).c()
    assert lib.moe_layout(ctypes.byref(bad), P(FAKE), ctypes.byref(b), None, 0, None) == moe.MOE_ERR_SHAPE
    nb = _bufs(moe)
    nb.status = None
    assert lib.moe_layout(ctypes.byref(d), P(FAKE), ctypes.byref(nb), None, 0, None) == moe.MOE_ERR_NULL
    mb = _bufs(moe, misalign="pos")
    assert lib.moe_layout(ctypes.byref(d), P(FAKE), ctypes.byref(mb), None, 0, None) == moe.MOE_ERR_ALIGN
    big = moe.LayoutDesc(8192, 8, 256, 8).c()
    need = lib.moe_layout_workspace_bytes(ctypes.byref(big))
    assert need > 0
    assert lib.moe_layout(ctypes.byref(big), P(FAKE), ctypes.byref(b), None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_layout(ctypes.byref(big), P(FAKE), ctypes.byref(b), P(FAKE), need - 4, None) == \
        moe.MOE_ERR_WORKSPACE


def test_dispatch_combine_argument_errors(moe):
    lib = moe.lib()
    P = ctypes.c_void_p
    d = moe.LayoutDesc(64, 2, 8, 2).c()
    b = _bufs(moe)
    x = P(FAKE)
    # dispatch: H not a multiple of 8, fp8 needs H % 128 == 0 and scales
    assert lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), x, 100, None, None, 0, x, None, None, None) == \
        moe.MOE_ERR_SHAPE
    assert lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), x, 136, None, None, 1, x, x, None, None) == \
        moe.MOE_ERR_SHAPE
    assert lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), x, 256, None, None, 1, x, None, None, None) == \
        moe.MOE_ERR_NULL
    assert lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), None, 256, None, None, 0, x, None, None, None) == \
        moe.MOE_ERR_NULL
    assert lib.moe_dispatch(ctypes.byref(d), ctypes.byref(b), P(FAKE + 8), 256, None, None, 0, x, None, None,
                            None) == moe.MOE_ERR_ALIGN
    assert lib.moe_dispatch(None, ctypes.byref(b), x, 256, None, None, 0, x, None, None, None) == moe.MOE_ERR_NULL
    # combine
    assert lib.moe_combine(ctypes.byref(d), ctypes.byref(b), x, 12, None, None, x, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_combine(ctypes.byref(d), ctypes.byref(b), None, 256, None, None, x, None) == moe.MOE_ERR_NULL
    assert lib.moe_combine(ctypes.byref(d), ctypes.byref(b), x, 256, None, P(FAKE + 4), x, None) == \
        moe.MOE_ERR_ALIGN
    assert lib.moe_combine(ctypes.byref(d), None, x, 256, None, None, x, None) == moe.MOE_ERR_NULL
    # an empty batch is a no-op
    e = moe.LayoutDesc(0, 2, 8, 2).c()
    assert lib.moe_dispatch(ctypes.byref(e), ctypes.byref(b), None, 256, None, None, 0, None, None, None, None) == \
        moe.MOE_OK
    assert lib.moe_combine(ctypes.byref(e), ctypes.byref(b), None, 256, None, None, None, None) == moe.MOE_OK


def test_zero_padding_argument_errors(moe):
    """moe_zero_padding rejects bad arguments before any launch."""
    lib = moe.lib()
    P = ctypes.c_void_p
    d = moe.LayoutDesc(64, 2, 8, 2, moe.MOE_PAD_CAPACITY, 20).c()
    b = _bufs(moe)
    assert lib.moe_zero_padding(None, ctypes.byref(b), 256, 0, P(FAKE), None, None) == moe.MOE_ERR_NULL
    assert lib.moe_zero_padding(ctypes.byref(d), None, 256, 0, P(FAKE), None, None) == moe.MOE_ERR_NULL
    assert lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), 12, 0, P(FAKE), None, None) == moe.MOE_ERR_SHAPE
    assert lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), 264, 1, P(FAKE), P(FAKE), None) == \
        moe.MOE_ERR_SHAPE                                            # FP8 needs H % 128 == 0
    assert lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), 256, 1, P(FAKE), None, None) == moe.MOE_ERR_NULL
    assert lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), 256, 0, None, None, None) == moe.MOE_ERR_NULL
    assert lib.moe_zero_padding(ctypes.byref(d), ctypes.byref(b), 256, 0, P(FAKE + 8), None, None) == \
        moe.MOE_ERR_ALIGN
    e = moe.LayoutDesc(0, 2, 8, 2).c()                               # empty batch: nothing to do
    assert lib.moe_zero_padding(ctypes.byref(e), ctypes.byref(b), 256, 0, None, None, None) == moe.MOE_OK


def test_balanced_workspace_rule(moe):
    """The balanced layout needs no scratch up to 32K entries (one launch) and
    reports MOE_ERR_WORKSPACE above that when none is given.  No launch."""
    assert moe.moe_layout_balanced_workspace_bytes(moe.LayoutDesc(4096, 8, 256, 8), 16) == 0
    big = moe.LayoutDesc(4097, 8, 256, 8)
    need = moe.moe_layout_balanced_workspace_bytes(big, 16)
    assert need >= 2 * 4097 * 8 * 4          # the plain layout's pos and src
    lib = moe.lib()
    P = ctypes.c_void_p
    d, b = big.c(), _bufs(moe)
    bb = moe.moe_balance_bufs(FAKE, FAKE + (1 << 16))
    args = (ctypes.byref(d), 16, P(FAKE), ctypes.byref(b), ctypes.byref(bb))
    assert lib.moe_layout_balanced(*args, None, 0, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_layout_balanced(*args, P(FAKE), need - 256, None) == moe.MOE_ERR_WORKSPACE
    assert lib.moe_layout_balanced(*args, P(FAKE + 16), need, None) == moe.MOE_ERR_ALIGN


def test_cu_range_stream_null_output(moe):
    assert moe.lib().moe_stream_create_cu_range(0, 8, None) == moe.MOE_ERR_NULL
    assert moe.lib().moe_stream_create_cu_limited(8, None) == moe.MOE_ERR_NULL


def test_status_strings(moe):
    for s in range(6):
        assert moe.moe_status_str(s).startswith("MOE_")
    assert moe.moe_status_str(99) == "unknown moe_status"


CEIL_HEADER = os.path.join(ROOT, "include", "moe_ceilings.h")


def test_ceiling_library_exports_and_rejects_bad_arguments():
    """The pattern-ceiling library exports every call its header declares and
    refuses bad shapes and misaligned pointers before any launch."""
    from combine_moe_layout_02_amd.build import CEIL_LIB
    if not os.path.exists(CEIL_LIB):
        import __graft_entry__
        __graft_entry__.build()
    text = re.sub(r"/\*.*?\*/", "", open(CEIL_HEADER).read(), flags=re.S)
    names = sorted(set(re.findall(r"\b(moe_ceiling_[a-z_0-9]+)\s*\(", text)))
    assert names == ["moe_ceiling_gather", "moe_ceiling_gather_persistent", "moe_ceiling_gather_policy",
                     "moe_ceiling_read", "moe_ceiling_scatter", "moe_ceiling_scatter_rows", "moe_ceiling_write"]
    import bench
    L = bench.ceiling_lib()
    for n in names:
        assert getattr(L, n) is not None
    ERR = 1
    P = ctypes.c_void_p
    A = FAKE
    assert L.moe_ceiling_read(None, 1 << 20, 1, 1, 0, P(A), None) == ERR
    assert L.moe_ceiling_read(P(A + 4), 1 << 20, 1, 1, 0, P(A), None) == ERR        # misaligned
    assert L.moe_ceiling_read(P(A), 1000, 1, 1, 0, P(A), None) == ERR                 # not whole KiB
    assert L.moe_ceiling_read(P(A), 1 << 20, 3, 1, 0, P(A), None) == ERR              # 3 vectors per lane
    assert L.moe_ceiling_read(P(A), 1 << 20, 1, 1, 2, P(A), None) == ERR              # unknown load kind
    assert L.moe_ceiling_read(P(A), 3 << 10, 1, 2, 0, P(A), None) == ERR              # 3 KiB over 2-wave groups
    assert L.moe_ceiling_write(P(A), 1 << 20, 1, 17, 0, None) == ERR                  # too many waves
    assert L.moe_ceiling_write(P(A), 1 << 20, 1, 1, 3, None) == ERR                   # unknown store kind
    assert L.moe_ceiling_scatter(P(A), 8, 3000, 8, P(A), P(A), 1024, None, 1, None) == ERR   # row ratio
    assert L.moe_ceiling_scatter(P(A), 8, 1536, 8, P(A), P(A), 1536, None, 1, None) == ERR   # not whole KiB
    assert L.moe_ceiling_scatter(P(A), 8, 2048, 3, P(A), P(A), 1024, None, 1, None) == ERR   # K = 3
    assert L.moe_ceiling_scatter(P(A), 8, 6144, 8, P(A), P(A), 3072, None, 2, None) == ERR   # 3 chunks in pairs
    assert L.moe_ceiling_scatter(P(A), 8, 4096, 8, P(A), P(A), 4096, None, 5, None) == ERR   # 5 waves
    assert L.moe_ceiling_gather(P(A), 8, 3072, 8, P(A), 2, 0, P(A), None) == ERR         # 3 KiB in 2 KiB chunks
    assert L.moe_ceiling_gather(P(A), 0, 1024, 8, P(A), 1, 0, P(A), None) == ERR         # empty
    assert L.moe_ceiling_gather(P(A), 8, 1024, 8, None, 1, 0, P(A), None) == ERR         # no rows


def test_ceiling_persistent_gather_rejects_bad_arguments():
    import bench
    L = bench.ceiling_lib()
    P = ctypes.c_void_p
    A = FAKE
    assert L.moe_ceiling_gather_persistent(P(A), 8, 1024, 8, P(A), 0, 1, 2, P(A), None) == 1    # no groups
    assert L.moe_ceiling_gather_persistent(P(A), 8, 1024, 8, P(A), 4, 5, 2, P(A), None) == 1    # 5 waves
    assert L.moe_ceiling_gather_persistent(P(A), 8, 1024, 7, P(A), 4, 1, 2, P(A), None) == 1    # K = 7
    assert L.moe_ceiling_gather_persistent(P(A), 8, 1536, 8, P(A), 4, 1, 2, P(A), None) == 1    # 1.5 KiB rows


def test_ceiling_scatter_rows_rejects_bad_arguments():
    import bench
    L = bench.ceiling_lib()
    P = ctypes.c_void_p
    A = FAKE
    assert L.moe_ceiling_scatter_rows(P(A), 8, 2048, 7, P(A), P(A), 1024, None, None) == 1       # K = 7
    assert L.moe_ceiling_scatter_rows(P(A), 8, 3072, 8, P(A), P(A), 1024, None, None) == 1       # row ratio
    assert L.moe_ceiling_scatter_rows(P(A), 8, 131072, 8, P(A), P(A), 131072, None, None) == 1   # row > 64 KiB


def test_ceiling_gather_policy_rejects_bad_arguments():
    import bench
    L = bench.ceiling_lib()
    P = ctypes.c_void_p
    A = FAKE
    assert L.moe_ceiling_gather_policy(P(A), 8, 1024, 8, P(A), 1, P(A), None) == 1    # policy 1 not swept
    assert L.moe_ceiling_gather_policy(P(A), 8, 1024, 6, P(A), 2, P(A), None) == 1    # K = 6
