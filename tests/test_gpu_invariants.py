"""GPU invariants of the tensor-parallel Linear on random-normal inputs.

These identities hold for any data, so they are checked bit for bit on
N(0,1) x N(0, 0.02^2) inputs, where rounding differs from element to element
and an accumulation-order difference would show:

  * repeated calls give identical bits (deterministic kernels and fold);
  * column-parallel with P shards equals P = 1 (the concatenation of the
    shard products is the dense product, "模型并行", "Column parallel"), and
    the TP_Y_SHARDS blocks are the column blocks of TP_Y_CONCAT;
  * row-parallel with P = 1 equals column-parallel with P = 1;
  * TP_ROW_FUSED equals TP_ROW_SUM (the fold inside the GEMM adds the same
    fp32 partials in the same order), both where the library picks the way
    to fold and with every shape a fused kernel takes sent to it
    (TPLINEAR_ROW_FOLD=gemm), and then leaves the workspace untouched on the
    decode shapes;
  * TP_ROW_SCATTER slices are the row blocks of TP_ROW_SUM, with and without
    gaps between the slices;
  * nothing outside an output view is written (guard cells keep their bits);
  * K = 0 gives +0 everywhere (an empty sum), in every mode.
"""
import numpy as np
import pytest
import torch

import synth
import tensor_linear_amd as tl
from gpu_util import DEV, FOLD_POLICIES, bf16_dev, f32_dev, bits, row_fold, workspace

pytestmark = pytest.mark.gpu

# (label, M, K, N, P, dtype): each reaches a different kernel for the column
# and/or the row GEMM (K/P, M and the tile count decide: skinny for M <= 48,
# for K/P % 64 == 0 the narrow kernel when the 256 x 256 tiles would fill at
# most half of the CUs -- 128 x 128 tiles when those fit in one pass, 128 x 64
# when they would fill at most half of it, else 256 x 128 -- and the 256 x 256
# tile kernel otherwise, the generic kernel
# for other K and for fp32).  Column P shards against P = 1 compares the
# 256 x 256 tile kernel with the 256 x 128 narrow tiles on "tile-ragged".
SHAPES = [
    ("narrow", 300, 1024, 1024, 8, "bf16"),          # column 128 x 64 tiles, row 128 x 128
    ("narrow-ragged", 257, 512, 520, 4, "bf16"),
    ("narrow256", 520, 1024, 2048, 4, "bf16"),       # row partials of 4 shards: 256 x 128 tiles
    ("tile-ragged", 1100, 1024, 4224, 16, "bf16"),   # 160 / 1360 256 x 256 tiles
    ("skinny-m1", 1, 2048, 1000, 8, "bf16"),
    ("skinny-m16", 16, 4160, 1000, 8, "bf16"),   # K/P = 520: ragged last stage
    ("skinny-m33", 33, 2048, 4096, 8, "bf16"),
    ("skinny-m48", 48, 1536, 264, 3, "bf16"),
    ("narrow-m64", 64, 1536, 264, 3, "bf16"),
    ("generic-bf16", 130, 576, 520, 8, "bf16"),  # row K/P = 72
    ("generic-f32", 70, 96, 48, 4, "f32"),
]

NAN16 = 0x7FC1          # guard pattern (a NaN no kernel produces from finite data)
NAN32 = 0x7FC00011


def _inputs(M, K, N, dt, seed):
    if dt == "bf16":
        X = bf16_dev(synth.normal_bf16(seed, (M, K), synth.SIGMA_X))
        W = bf16_dev(synth.normal_bf16(seed + 1, (N, K), synth.SIGMA_W))
    else:
        X = f32_dev(synth.normal_f32(seed, (M, K), synth.SIGMA_X))
        W = f32_dev(synth.normal_f32(seed + 1, (N, K), synth.SIGMA_W))
    return X, W


def _tdt(dt):
    return torch.bfloat16 if dt == "bf16" else torch.float32


def _guarded(shape, dtype, lead=40, trail=40):
    """A flat buffer of guard bits; returns (buffer, element offset)."""
    n = int(np.prod(shape)) + lead + trail
    if dtype == torch.bfloat16:
        buf = torch.full((n,), NAN16, dtype=torch.int16, device=DEV).view(torch.bfloat16)
    else:
        buf = torch.full((n,), NAN32, dtype=torch.int32, device=DEV).view(torch.float32)
    return buf, lead


def _guard_ok(buf, mask):
    """Every element outside `mask` still holds the guard pattern."""
    b = bits(buf)
    pat = NAN16 if buf.dtype == torch.bfloat16 else NAN32
    return bool(np.all(b[~mask] == pat))


def _row_y(X, W, P, mode, dt, M, N):
    Y = torch.empty((M, N), dtype=_tdt(dt), device=DEV)
    tl.tp_linear_row(X, W, Y, P, mode, workspace(mode, M, N, P))
    return Y


def _col_y(X, W, P, dt, M, N):
    Y = torch.empty((M, N), dtype=_tdt(dt), device=DEV)
    tl.tp_linear_column(X, W, Y, P)
    return Y


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_repeat_calls_bitwise(shape):
    label, M, K, N, P, dt = shape
    print(f"{label}: M={M} K={K} N={N} P={P} {dt}", flush=True)
    X, W = _inputs(M, K, N, dt, 900)
    a = _col_y(X, W, P, dt, M, N)
    b = torch.full_like(a, 3.0)
    tl.tp_linear_column(X, W, b, P)
    assert np.array_equal(bits(a), bits(b)), "column"
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
        a = _row_y(X, W, P, mode, dt, M, N)
        # second call: stale output and a workspace holding old partials
        ws = workspace(mode, M, N, P)
        tl.tp_linear_row(X, W, a.clone(), P, mode, ws)
        b = torch.full_like(a, -7.0)
        tl.tp_linear_row(X, W, b, P, mode, ws)
        assert np.array_equal(bits(a), bits(b)), f"row mode {mode}"


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_column_shards_equal_dense(shape):
    label, M, K, N, P, dt = shape
    print(f"{label}: M={M} K={K} N={N} P={P} {dt}", flush=True)
    X, W = _inputs(M, K, N, dt, 910)
    dense = bits(_col_y(X, W, 1, dt, M, N))
    for p in sorted({2, P}):
        if N % p:
            continue
        assert np.array_equal(bits(_col_y(X, W, p, dt, M, N)), dense), f"P={p} concat"
        Ys = torch.empty((p, M, N // p), dtype=_tdt(dt), device=DEV)
        tl.tp_linear_column(X, W, Ys, p, tl.TP_Y_SHARDS)
        for i in range(p):
            assert np.array_equal(bits(Ys[i]), dense[:, i * (N // p):(i + 1) * (N // p)]), \
                f"P={p} shard block {i}"


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_row_p1_equals_column_p1(shape):
    label, M, K, N, P, dt = shape
    X, W = _inputs(M, K, N, dt, 920)
    col = bits(_col_y(X, W, 1, dt, M, N))
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
        assert np.array_equal(bits(_row_y(X, W, 1, mode, dt, M, N)), col), f"mode {mode}"


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
def test_fused_equals_sum(shape):
    label, M, K, N, P, dt = shape
    X, W = _inputs(M, K, N, dt, 930)
    for p in sorted({1, 3, P}):
        if K % p:
            continue
        s = bits(_row_y(X, W, p, tl.TP_ROW_SUM, dt, M, N))
        for policy in FOLD_POLICIES:
            with row_fold(policy):
                f = bits(_row_y(X, W, p, tl.TP_ROW_FUSED, dt, M, N))
            assert np.array_equal(s, f), f"P={p} {policy}"


@pytest.mark.parametrize("M,K,N,P", [(1, 2048, 1000, 8), (16, 4160, 1000, 8),
                                     (48, 1536, 264, 3)])
def test_fused_decode_leaves_workspace(M, K, N, P):
    """The fused decode path needs no partials in memory (sent to it at
    every decode shape)."""
    X, W = _inputs(M, K, N, "bf16", 940)
    nbytes = tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, M, N, P)
    ws = torch.full((nbytes // 4,), NAN32, dtype=torch.int32, device=DEV)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    with row_fold("gemm"):
        tl.tp_linear_row(X, W, Y, P, tl.TP_ROW_FUSED, ws.view(torch.uint8))
    torch.cuda.synchronize()
    assert bool((ws == NAN32).all()), "workspace written"
    assert not torch.isnan(Y.float()).any()


@pytest.mark.parametrize("M,K,N,P", [(64, 2048, 1000, 8), (512, 1024, 1024, 8),
                                     (258, 576, 520, 3)])
def test_scatter_equals_sum(M, K, N, P):
    X, W = _inputs(M, K, N, "bf16", 950)
    ref = bits(_row_y(X, W, P, tl.TP_ROW_SUM, "bf16", M, N))
    got = bits(_row_y(X, W, P, tl.TP_ROW_SCATTER, "bf16", M, N))
    assert np.array_equal(got, ref), "contiguous slices"
    # slices in separate places: slice j at element j*stride, rows M/P
    s = M // P
    stride = s * N + 1000
    buf, off = _guarded((P * stride,), torch.bfloat16)
    Y0 = buf[off: off + s * N].view(s, N)
    tl.tp_linear_row(X, W, Y0, P, tl.TP_ROW_SCATTER, workspace(tl.TP_ROW_SCATTER, M, N, P),
                     y_slice_stride=stride)
    b = bits(buf)
    mask = np.zeros(b.shape, dtype=bool)
    for j in range(P):
        lo = off + j * stride
        assert np.array_equal(b[lo: lo + s * N].reshape(s, N), ref[j * s:(j + 1) * s]), \
            f"slice {j}"
        mask[lo: lo + s * N] = True
    assert _guard_ok(buf, mask), "wrote between slices"


@pytest.mark.parametrize("shape", SHAPES, ids=[s[0] for s in SHAPES])
@pytest.mark.parametrize("col0", [8, 3])
def test_guard_cells(shape, col0):
    """Outputs as views into bigger buffers: leading dim N + 24, first column
    col0 (8 keeps 16-byte alignment, 3 does not)."""
    label, M, K, N, P, dt = shape
    X, W = _inputs(M, K, N, dt, 960)
    tdt = _tdt(dt)
    ld = N + 24
    dense = bits(_col_y(X, W, P, dt, M, N))
    rsum = bits(_row_y(X, W, P, tl.TP_ROW_SUM, dt, M, N)) if K % P == 0 else None

    def view(buf, off, rows):
        return buf[off: off + rows * ld].view(rows, ld)[:, col0: col0 + N]

    def mask_of(n, off, rows):
        m = np.zeros(n, dtype=bool)
        for r in range(rows):
            m[off + r * ld + col0: off + r * ld + col0 + N] = True
        return m

    buf, off = _guarded((M * ld,), tdt)
    Y = view(buf, off, M)
    tl.tp_linear_column(X, W, Y, P)
    assert np.array_equal(bits(Y), dense)
    assert _guard_ok(buf, mask_of(buf.numel(), off, M)), "column wrote outside Y"
    if rsum is None:
        return
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
        buf, off = _guarded((M * ld,), tdt)
        Y = view(buf, off, M)
        tl.tp_linear_row(X, W, Y, P, mode, workspace(mode, M, N, P))
        assert np.array_equal(bits(Y), rsum), f"mode {mode}"
        assert _guard_ok(buf, mask_of(buf.numel(), off, M)), f"mode {mode} wrote outside Y"
    # fp32 partials: P blocks of M rows, each row ld wide
    buf, off = _guarded((P * M * ld,), torch.float32)
    Yp = buf[off: off + P * M * ld].view(P, M, ld)[:, :, col0: col0 + N]
    tl.tp_linear_row(X, W, Yp, P, tl.TP_ROW_PARTIAL)
    assert _guard_ok(buf, mask_of(buf.numel(), off, P * M)), "partials wrote outside"
    assert not torch.isnan(Yp).any()


@pytest.mark.parametrize("M,N,P", [(300, 512, 8), (16, 1000, 8), (5, 24, 3)])
def test_zero_k(M, N, P):
    """K = 0: an empty sum, so every output is +0 (and nothing is read)."""
    for dt in ("bf16", "f32"):
        tdt = _tdt(dt)
        X = torch.empty((M, 0), dtype=tdt, device=DEV)
        W = torch.empty((N, 0), dtype=tdt, device=DEV)
        Y = torch.full((M, N), 7.0, dtype=tdt, device=DEV)
        tl.tp_linear_column(X, W, Y, P)
        assert not bits(Y).any(), "column"
        for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
            Y.fill_(7.0)
            tl.tp_linear_row(X, W, Y, P, mode, workspace(mode, M, N, P))
            assert not bits(Y).any(), f"row mode {mode}"
