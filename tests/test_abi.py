"""CPU tests of the C ABI: the library loads without a GPU, exports every
function include/tplinear.h declares, maps placements to views exactly as
the oracle's integer index maps do, and rejects every bad argument on the
host before queuing any GPU work.  No call here reaches a kernel."""
import ctypes
import os
import re

import pytest

import oracle
import tensor_linear_amd as tl

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _declared_functions():
    with open(os.path.join(ROOT, "include", "tplinear.h")) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(tp_[a-z_]+)\s*\(", text)))


def test_every_declared_function_is_exported():
    declared = _declared_functions()
    assert set(declared) == set(tl.EXPORTS)
    lib = ctypes.CDLL(tl.LIB_PATH)
    for name in declared:
        assert hasattr(lib, name), name


def test_clock_probe_library_loads():
    # The bench's shader-clock probe lives in a library of its own; it must
    # load without a GPU and export its one entry point.
    path = os.path.join(ROOT, "tensor_linear_amd", "libtplclock.so")
    if not os.path.exists(path):
        pytest.skip("libtplclock.so not built")
    lib = ctypes.CDLL(path)
    assert hasattr(lib, "tp_clock_probe")


def test_status_strings():
    for s in range(9):
        assert tl.tp_status_str(s).startswith("TP_")
    assert "unknown" in tl.tp_status_str(99)
    assert tl.tp_version() >= 100


# ---- tp_shard_layout against the oracle's index maps (bit-exact) ----------

@pytest.mark.parametrize("R,C,extra", [(1, 1, 0), (4, 4, 0), (6, 10, 3), (8, 3, 1),
                                       (12, 12, 5), (16, 64, 0)])
def test_layout_matches_oracle(R, C, extra):
    ld = C + extra
    for kind in (tl.TP_SHARD, tl.TP_REPLICATE, tl.TP_PARTIAL):
        dims = (0, 1, -1, -2) if kind == tl.TP_SHARD else (0,)
        for dim in dims:
            L = R if dim in (0, -2) else C
            for P in range(1, min(L, 16) + 1):
                if kind == tl.TP_SHARD and L % P:
                    with pytest.raises(tl.TPError) as e:
                        tl.tp_shard_layout(R, C, ld, kind, dim, P)
                    assert e.value.status == tl.TP_ERR_INDIVISIBLE
                    continue
                got = tl.tp_shard_layout(R, C, ld, kind, dim, P)
                want = oracle.expected_views(R, C, ld, kind, dim, P)
                assert got == want, (kind, dim, P)


def test_layout_printed_example():
    # DTensor API page, distribute_tensor: 4x4 arange, Shard(0) over 2 ->
    # rows 0-1 and rows 2-3.
    import numpy as np
    A = np.arange(16).reshape(4, 4)
    views = tl.tp_shard_layout(4, 4, 4, tl.TP_SHARD, 0, 2)
    flat = A.reshape(-1)
    got = [flat[off:off + r * ld].reshape(r, ld)[:, :c] for off, r, c, ld, _, _ in views]
    assert np.array_equal(got[0], [[0, 1, 2, 3], [4, 5, 6, 7]])
    assert np.array_equal(got[1], [[8, 9, 10, 11], [12, 13, 14, 15]])
    # weight (1024, 4096), Shard(1) over 4 -> (1024, 1024) each
    assert all((r, c) == (1024, 1024) for _, r, c, _, _, _ in
               tl.tp_shard_layout(1024, 4096, 4096, tl.TP_SHARD, 1, 4))


def test_layout_errors():
    lib = tl.lib
    views = (tl.tp_view * 4)()
    pl = tl.tp_placement(tl.TP_SHARD, 0)
    assert lib.tp_shard_layout(4, 4, 4, pl, 2, None) == tl.TP_ERR_NULL
    assert lib.tp_shard_layout(-1, 4, 4, pl, 2, views) == tl.TP_ERR_SHAPE
    assert lib.tp_shard_layout(4, 4, 3, pl, 2, views) == tl.TP_ERR_SHAPE
    assert lib.tp_shard_layout(4, 4, 4, pl, 0, views) == tl.TP_ERR_SHAPE
    assert lib.tp_shard_layout(4, 4, 4, pl, 65, views) == tl.TP_ERR_SHAPE
    assert lib.tp_shard_layout(4, 4, 4, tl.tp_placement(7, 0), 2, views) == tl.TP_ERR_PLACEMENT
    assert lib.tp_shard_layout(4, 4, 4, tl.tp_placement(tl.TP_SHARD, 2), 2, views) == \
        tl.TP_ERR_PLACEMENT
    assert lib.tp_shard_layout(4, 4, 4, tl.tp_placement(tl.TP_SHARD, -3), 2, views) == \
        tl.TP_ERR_PLACEMENT
    assert lib.tp_shard_layout(5, 4, 4, pl, 2, views) == tl.TP_ERR_INDIVISIBLE
    assert lib.tp_shard_layout(0, 0, 0, pl, 4, views) == tl.TP_OK


# ---- host-side argument checks of the compute entry points ---------------
# Fake but non-null addresses: every call below must be rejected (or be an
# empty problem) before anything is queued, so no address is dereferenced.

FX, FW, FY, FWS = 0x100000, 0x200000, 0x300000, 0x400000


def col(**kw):
    a = dict(X=FX, ldx=8, W=FW, ldw=8, Y=FY, ldy=12, y_mode=tl.TP_Y_CONCAT, M=3, N=12, K=8,
             P=4, dtype=tl.TP_BF16, stream=None)
    a.update(kw)
    return tl.lib.tp_linear_column(a["X"], a["ldx"], a["W"], a["ldw"], a["Y"], a["ldy"],
                                   a["y_mode"], a["M"], a["N"], a["K"], a["P"], a["dtype"],
                                   a["stream"])


def row(**kw):
    a = dict(X=FX, ldx=8, W=FW, ldw=8, Y=FY, ldy=12, ss=0, mode=tl.TP_ROW_SUM, ws=FWS,
             wsb=1 << 20, M=4, N=12, K=8, P=4, dtype=tl.TP_BF16, stream=None)
    a.update(kw)
    return tl.lib.tp_linear_row(a["X"], a["ldx"], a["W"], a["ldw"], a["Y"], a["ldy"], a["ss"],
                                a["mode"], a["ws"], a["wsb"], a["M"], a["N"], a["K"], a["P"],
                                a["dtype"], a["stream"])


def red(**kw):
    a = dict(p=FWS, ss=48, ldp=12, Y=FY, ldy=12, yss=0, scatter=0, M=4, N=12, P=4,
             dtype=tl.TP_BF16, stream=None)
    a.update(kw)
    return tl.lib.tp_shard_reduce(a["p"], a["ss"], a["ldp"], a["Y"], a["ldy"], a["yss"],
                                  a["scatter"], a["M"], a["N"], a["P"], a["dtype"], a["stream"])


def test_column_errors():
    assert col(X=None) == tl.TP_ERR_NULL
    assert col(W=None) == tl.TP_ERR_NULL
    assert col(Y=None) == tl.TP_ERR_NULL
    assert col(M=-1) == tl.TP_ERR_SHAPE
    assert col(K=-1) == tl.TP_ERR_SHAPE
    assert col(P=0) == tl.TP_ERR_SHAPE
    assert col(P=65) == tl.TP_ERR_SHAPE
    assert col(ldx=7) == tl.TP_ERR_SHAPE
    assert col(ldw=7) == tl.TP_ERR_SHAPE
    assert col(ldy=11) == tl.TP_ERR_SHAPE                       # concat needs ldy >= N
    assert col(ldy=2, y_mode=tl.TP_Y_SHARDS) == tl.TP_ERR_SHAPE  # shards need ldy >= N/P
    assert col(N=10) == tl.TP_ERR_INDIVISIBLE
    assert col(dtype=2) == tl.TP_ERR_DTYPE
    assert col(y_mode=5) == tl.TP_ERR_MODE
    # empty problems are valid and queue nothing
    assert col(M=0) == tl.TP_OK
    assert col(N=0) == tl.TP_OK
    assert col(M=0, X=None, W=None, Y=None) == tl.TP_OK


def test_row_errors():
    need = tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 4, 12, 4)
    assert need >= 4 * 4 * 12 * 4
    assert row(X=None) == tl.TP_ERR_NULL
    assert row(Y=None) == tl.TP_ERR_NULL
    assert row(P=0) == tl.TP_ERR_SHAPE
    assert row(ldy=11) == tl.TP_ERR_SHAPE
    assert row(ss=-1, mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_SHAPE
    # slices that would overlap: a nonzero stride below (M/P - 1)*ldy + N
    assert row(ss=11, mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_SHAPE            # M/P = 1
    assert row(ss=23, M=8, mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_SHAPE      # M/P = 2
    assert row(ss=23, M=8, ldy=16, mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_SHAPE
    assert row(ss=11, mode=tl.TP_ROW_SCATTER, M=0) == tl.TP_OK           # empty: nothing written
    assert row(K=10, ldx=10, ldw=10) == tl.TP_ERR_INDIVISIBLE
    assert row(M=6, mode=tl.TP_ROW_SCATTER) == tl.TP_ERR_INDIVISIBLE
    assert row(dtype=7) == tl.TP_ERR_DTYPE
    assert row(mode=4) == tl.TP_ERR_MODE
    assert row(mode=-1) == tl.TP_ERR_MODE
    assert row(ws=None) == tl.TP_ERR_WORKSPACE
    assert row(wsb=need - 1) == tl.TP_ERR_WORKSPACE
    assert row(ws=FWS + 4) == tl.TP_ERR_WORKSPACE              # not 256-byte aligned
    assert row(mode=tl.TP_ROW_FUSED, wsb=need - 1) == tl.TP_ERR_WORKSPACE
    assert row(M=0) == tl.TP_OK
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_PARTIAL, 4, 12, 4) == 0
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 4, 12, 0) == 0
    fused = tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, 16, 8192, 8)
    assert fused == tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 16, 8192, 8) >= 8 * 16 * 8192 * 4


def test_reduce_errors():
    assert red(p=None) == tl.TP_ERR_NULL
    assert red(Y=None) == tl.TP_ERR_NULL
    assert red(P=0) == tl.TP_ERR_SHAPE
    assert red(ldp=11) == tl.TP_ERR_SHAPE
    assert red(ldy=11) == tl.TP_ERR_SHAPE
    assert red(ss=-1) == tl.TP_ERR_SHAPE
    assert red(dtype=3) == tl.TP_ERR_DTYPE
    assert red(scatter=2) == tl.TP_ERR_MODE
    assert red(scatter=1, M=6) == tl.TP_ERR_INDIVISIBLE
    assert red(scatter=1, yss=11) == tl.TP_ERR_SHAPE                     # overlapping slices
    assert red(scatter=1, yss=23, M=8, ss=96) == tl.TP_ERR_SHAPE
    assert red(M=0) == tl.TP_OK


def test_oversized_extents_rejected():
    # Sizes whose element counts pass 2^60 are rejected before any size
    # arithmetic can wrap: in particular a wrapped workspace size must never
    # let a too-small workspace through.
    big = 1 << 31
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, big, big, 8) == 0
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 1 << 62, 1 << 62, 8) == 0
    assert row(M=big, N=big, ldy=big) == tl.TP_ERR_SHAPE
    assert row(M=1 << 62, N=1 << 62, ldy=1 << 62) == tl.TP_ERR_SHAPE
    assert row(M=4, N=12, ldy=12, ldx=1 << 62, ldw=8) == tl.TP_ERR_SHAPE
    assert row(mode=tl.TP_ROW_SCATTER, ss=1 << 62) == tl.TP_ERR_SHAPE
    assert col(M=1 << 40, ldx=1 << 40) == tl.TP_ERR_SHAPE
    assert col(M=1 << 40, ldy=1 << 40) == tl.TP_ERR_SHAPE
    assert red(ss=1 << 62) == tl.TP_ERR_SHAPE
    assert red(M=1 << 40, ldp=1 << 40) == tl.TP_ERR_SHAPE
    views = (tl.tp_view * 4)()
    assert tl.lib.tp_shard_layout(1 << 40, 4, 1 << 40, tl.tp_placement(tl.TP_SHARD, 0), 2,
                                  views) == tl.TP_ERR_SHAPE
    assert tl.lib.tp_shard_layout(1 << 31, 4, 1 << 30, tl.tp_placement(tl.TP_PARTIAL, 0), 4,
                                  views) == tl.TP_ERR_SHAPE
    # the largest accepted sizes still pass the checks (empty N: nothing queued)
    assert row(M=1 << 20, N=0, ldy=1) == tl.TP_OK


def test_workspace_zero_errors():
    assert tl.lib.tp_workspace_zero(None, 16, None) == tl.TP_ERR_NULL
    assert tl.lib.tp_workspace_zero(FWS, 6, None) == tl.TP_ERR_SHAPE
    assert tl.lib.tp_workspace_zero(None, 0, None) == tl.TP_OK


def test_binding_leading_dims():
    """The binding's (rows, cols, leading dim) of 2-D views, host only."""
    import torch
    buf = torch.zeros(4 * 1 * 40)
    parts = buf.view(4, 1, 40)[:, :, 3:19]          # [P, 1, N] cut from rows of 40
    assert tl._mat(parts[0], "Y")[1:] == (1, 16, 40)
    assert tl._mat(torch.zeros(1, 16), "Y")[1:] == (1, 16, 16)
    assert tl._mat(torch.zeros(5, 16)[:, :8], "Y")[1:] == (5, 8, 16)
    assert tl._mat(torch.zeros(0, 5), "Y")[1:] == (0, 5, 5)
    with pytest.raises(ValueError):
        tl._mat(torch.zeros(4, 6).t(), "Y")


def test_binding_rejects_host_tensors():
    """The kernels dereference device pointers: host tensors are refused by
    the binding before the library is called."""
    import torch
    bf = torch.bfloat16
    X, W, Y = torch.zeros(4, 8, dtype=bf), torch.zeros(12, 8, dtype=bf), torch.zeros(4, 12, dtype=bf)
    parts = torch.zeros(4, 4, 12)
    calls = [
        lambda: tl.tp_linear_column(X, W, Y, 4),
        lambda: tl.tp_linear_column_ex(X, W, Y, 4),
        lambda: tl.tp_linear_row(X, W, Y, 4, tl.TP_ROW_SUM, torch.zeros(1 << 12, dtype=torch.uint8)),
        lambda: tl.tp_linear_row_ex(X, W, parts, 4, tl.TP_ROW_PARTIAL),
        lambda: tl.tp_shard_reduce(parts, Y, 4),
        lambda: tl.tp_shard_reduce_ex(parts, Y, 4),
        lambda: tl.tp_embedding(torch.zeros(4, dtype=torch.int64), torch.zeros(4, 8, dtype=bf), 4,
                                E=W),
        lambda: tl.tp_workspace_zero(torch.zeros(16, dtype=torch.uint8)),
    ]
    for c in calls:
        with pytest.raises(ValueError, match="GPU tensor"):
            c()


def test_binding_rejects_misshaped_outputs():
    """The library writes exactly the output the sizes call for; the binding
    refuses an output tensor of another shape (too few rows, a narrower
    column view, a wrong block shape) or a slice buffer too small for P
    strided slices, before any device check or library call."""
    import torch
    bf, f32 = torch.bfloat16, torch.float32
    M, K, N, P = 8, 16, 12, 4
    X, W = torch.zeros(M, K, dtype=bf), torch.zeros(N, K, dtype=bf)
    parts = torch.zeros(P, M, N)
    Y = lambda *s: torch.zeros(*s, dtype=bf)                      # noqa: E731
    bad = [
        lambda: tl.tp_linear_column(X, W, Y(M - 1, N), P),
        lambda: tl.tp_linear_column(X, W, Y(M, N + 4)[:, :N - 1], P),
        lambda: tl.tp_linear_column(X, W, Y(P, M, N // P - 1), P, tl.TP_Y_SHARDS),
        lambda: tl.tp_linear_column(X, W, Y(P, M - 1, N // P), P, tl.TP_Y_SHARDS),
        lambda: tl.tp_linear_column_ex(X, torch.zeros(16, K, dtype=bf), Y(M, 16), P,
                                       act=tl.TP_ACT_SWIGLU),      # needs [M, 8]
        lambda: tl.tp_linear_column_ex(X, W, Y(M, N), P, bias=Y(N - 1)),
        lambda: tl.tp_linear_row(X, W, Y(M - 1, N), P, tl.TP_ROW_SUM),
        lambda: tl.tp_linear_row(X, W, Y(M, N - 1), P, tl.TP_ROW_FUSED),
        lambda: tl.tp_linear_row(X, W, torch.zeros(P, M, N - 1), P, tl.TP_ROW_PARTIAL),
        lambda: tl.tp_linear_row(X, W, torch.zeros(P - 1, M, N), P, tl.TP_ROW_PARTIAL),
        lambda: tl.tp_linear_row_ex(X, W, Y(M, N), P, bias=Y(N + 1)),
        # slice 0 of P strided slices: the buffer must reach the last slice
        lambda: tl.tp_linear_row(X, W, Y(P * 2 * N)[:2 * N].view(2, N), P,
                                 tl.TP_ROW_SCATTER, y_slice_stride=3 * N),
        lambda: tl.tp_linear_row(X, W, Y(M // P + 1, N), P, tl.TP_ROW_SCATTER,
                                 y_slice_stride=3 * N),
        lambda: tl.tp_shard_reduce(parts, Y(M, N + 1), P),
        lambda: tl.tp_shard_reduce(parts, Y(M - 1, N), P, scatter=1),
        lambda: tl.tp_shard_reduce(parts, Y(4 * N)[:2 * N].view(2, N), P, scatter=1,
                                   y_slice_stride=2 * N),
        lambda: tl.tp_shard_reduce_ex(parts, Y(M, N), P, bias=Y(N - 1)),
        lambda: tl.tp_embedding(torch.zeros(5, dtype=torch.int64), Y(4, 16), P, E=Y(10, 16)),
        lambda: tl.tp_embedding(torch.zeros(5, dtype=torch.int64), Y(5, 12), P, E=Y(10, 16)),
        lambda: tl.tp_embedding(torch.zeros(5, dtype=torch.int64), Y(P, 5, 3), P, E=Y(10, 16),
                                y_mode=tl.TP_Y_SHARDS),
    ]
    for i, c in enumerate(bad):
        with pytest.raises(ValueError, match="shape|storage") as e:
            c()
        assert "GPU tensor" not in str(e.value), i
    # correctly shaped host outputs pass the shape checks and reach the
    # device check (the slice buffer here holds all P slices exactly)
    ok = [
        lambda: tl.tp_linear_column(X, W, Y(M, N), P),
        lambda: tl.tp_linear_row(X, W, Y(P * 3 * N)[:2 * N].view(2, N), P, tl.TP_ROW_SCATTER,
                                 y_slice_stride=3 * N),
        lambda: tl.tp_shard_reduce(parts, Y(3 * 2 * N + 2 * N)[:2 * N].view(2, N), P,
                                   scatter=1, y_slice_stride=2 * N),
    ]
    for c in ok:
        with pytest.raises(ValueError, match="GPU tensor"):
            c()
    # an indivisible split is the library's status, also from the binding
    with pytest.raises(tl.TPError) as e:
        tl.tp_linear_column(X, torch.zeros(10, K, dtype=bf), Y(M, 10), P)
    assert e.value.status == tl.TP_ERR_INDIVISIBLE
    with pytest.raises(tl.TPError) as e:
        tl.tp_shard_reduce(torch.zeros(P, 6, N, dtype=f32), Y(6, N), P, scatter=1)
    assert e.value.status == tl.TP_ERR_INDIVISIBLE


def test_noalloc_rejects_before_any_device_call():
    """tp_linear_row_noalloc: a shape whose workspace would exceed the fixed
    per-GPU array is TP_ERR_WORKSPACE on the host; argument errors are the
    ones tp_linear_row reports.  Nothing here reaches a device."""
    lib = tl.lib

    def call(M, N, K, P, mode=tl.TP_ROW_SUM, ldy=None):
        return lib.tp_linear_row_noalloc(FX, K, FW, K, FY, N if ldy is None else ldy, 0, mode,
                                         M, N, K, P, tl.TP_BF16, None)
    cap = tl.TP_NOALLOC_SCRATCH_BYTES
    # 4096 x 4096 x 8 fp32 partials = 512 MiB > the array; TP_ROW_SUM always
    # folds them in a separate kernel, TP_ROW_FUSED and TP_ROW_SCATTER do at
    # a shard K of 8192 (too long for the fold inside the GEMM)
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, 4096, 4096, 8) > cap
    assert call(4096, 4096, 4096, 8) == tl.TP_ERR_WORKSPACE
    assert call(4096, 4096, 8 * 8192, 8, tl.TP_ROW_SCATTER) == tl.TP_ERR_WORKSPACE
    assert call(4096, 4096, 8 * 8192, 8, tl.TP_ROW_FUSED) == tl.TP_ERR_WORKSPACE
    # one partial element past the limit
    M = cap // (4 * 1024 * 8) + 1
    assert tl.tp_row_workspace_bytes(tl.TP_ROW_SUM, M, 1024, 8) > cap
    assert call(M, 1024, 64, 8) == tl.TP_ERR_WORKSPACE
    # argument errors as tp_linear_row
    assert call(4, 12, 8, 0) == tl.TP_ERR_SHAPE
    assert call(4, 12, 10, 4) == tl.TP_ERR_INDIVISIBLE
    assert call(4, 12, 8, 4, mode=9) == tl.TP_ERR_MODE
    assert call(4, 12, 8, 4, ldy=11) == tl.TP_ERR_SHAPE
    assert call(0, 12, 8, 4) == tl.TP_OK
