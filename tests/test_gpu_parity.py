"""GPU parity: the HIP path through the C ABI against the CPU oracle on the
same seeded inputs.

  * integer-valued inputs: every sum is exact in fp32, so every kernel and
    mode must match the oracle bit for bit (after the one rounding to the
    output type, done by the oracle's own RNE);
  * the shard fold on synthetic fp32 partials: bit-exact against the
    oracle's fp32 left fold + RNE;
  * N(0,1) x N(0, 0.02^2) inputs at the workload shapes with reduced M: rel L2
    <= 1e-2 and max abs <= 2e-2 sqrt(K) sx sw (bf16), rel L2 <= 1e-5 (fp32);
  * the worked example of the model-parallelism page (fp32).
"""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import (DEV, FOLD_POLICIES, bf16_dev, f32_dev, to_f64, bits, expected_bits, row_fold,
                      workspace, bf16_tol)

pytestmark = pytest.mark.gpu

DT = {"bf16": torch.bfloat16, "f32": torch.float32}


def _inputs_int(seed, M, K, N, dtype):
    """Integer-valued X [M,K] and W [N,K] on the device, plus fp64 copies
    with W in [in,out] orientation for the oracle."""
    X = synth.small_ints(seed, (M, K))
    W = synth.small_ints(seed + 1, (N, K))
    if dtype == torch.bfloat16:
        Xd, Wd = bf16_dev(synth.to_bf16_bits(X)), bf16_dev(synth.to_bf16_bits(W))
    else:
        Xd, Wd = f32_dev(X), f32_dev(W)
    return Xd, Wd, X.astype(np.float64), W.T.astype(np.float64)


def _run_all_modes(Xd, Wd, X64, Wio, M, K, N, P, dtype):
    """Run every column and row mode and compare bit for bit."""
    # column, concatenated
    Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column(Xd, Wd, Y, P, tl.TP_Y_CONCAT)
    ref = oracle.column_parallel_linear(X64, Wio, P)
    assert np.array_equal(bits(Y), expected_bits(ref, dtype)), "column concat"
    # column, shard blocks
    Ys = torch.full((P, M, N // P), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column(Xd, Wd, Ys, P, tl.TP_Y_SHARDS)
    for i, yi in enumerate(oracle.column_shards(X64, Wio, P)):
        assert np.array_equal(bits(Ys[i]), expected_bits(yi, dtype)), f"column shard {i}"
    if K % P:
        return
    # row partials (fp32)
    Yp = torch.full((P, M, N), float("nan"), dtype=torch.float32, device=DEV)
    tl.tp_linear_row(Xd, Wd, Yp, P, tl.TP_ROW_PARTIAL)
    for i, pi in enumerate(oracle.row_partials(X64, Wio, P)):
        assert np.array_equal(bits(Yp[i]), expected_bits(pi, torch.float32)), f"row partial {i}"
    ref = oracle.row_parallel_linear(X64, Wio, P)
    slices = oracle.reduce_scatter_rows(oracle.row_partials(X64, Wio, P), P) if M % P == 0 else None
    for policy in FOLD_POLICIES:
        with row_fold(policy):
            for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
                Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
                tl.tp_linear_row(Xd, Wd, Y, P, mode, workspace(mode, M, N, P))
                assert np.array_equal(bits(Y), expected_bits(ref, dtype)), f"row mode {mode} {policy}"
            if slices is None:
                continue
            Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
            tl.tp_linear_row(Xd, Wd, Y, P, tl.TP_ROW_SCATTER, workspace(tl.TP_ROW_SCATTER, M, N, P))
            s = M // P
            for j, sl in enumerate(slices):
                assert np.array_equal(bits(Y[j * s:(j + 1) * s]), expected_bits(sl, dtype)), \
                    f"scatter slice {j} {policy}"


# Tiny shapes (generic kernel): M in {1,2,3,5}, P in {1,2,3,4,8},
# N/P and K/P in {1,2,3,5}.
TINY = [(M, P, ns, ks) for M in (1, 2, 3, 5) for P in (1, 2, 3, 4, 8)
        for ns in (1, 2, 3, 5) for ks in (1, 2, 3, 5)]


@pytest.mark.parametrize("dt", ["bf16", "f32"])
def test_brute_force_tiny_bitwise(dt):
    dtype = DT[dt]
    for idx, (M, P, ns, ks) in enumerate(TINY):
        N, K = ns * P, ks * P
        Xd, Wd, X64, Wio = _inputs_int(100 + idx, M, K, N, dtype)
        _run_all_modes(Xd, Wd, X64, Wio, M, K, N, P, dtype)


# Shapes that reach the skinny (M <= 48), narrow (128 x 64, 128 x 128 and
# 256 x 128) and 256 x 256 tile kernels, with ragged M and N tails; integer
# inputs keep every sum exact.
ALIGNED = [
    (16, 8192 // 8 * 8, 256, 8),   # skinny, one m-block
    (1, 512, 64, 8),
    (17, 256, 192, 4),             # skinny, two m-blocks, ragged M
    (48, 1024, 512, 2),            # skinny, three m-blocks
    (40, 512, 4096 * 8, 8),        # 33-48 tokens on the tile order: column 128 x 128 tiles, row 256 x 256
    (64, 1024, 512, 2),            # 128 x 64 tiles, 64 tokens
    (65, 512, 512, 2),             # few tiles: 128 x 64 tiles, mostly-empty M tile
    (300, 512, 2 * 300, 2),        # 128 x 64 tiles, ragged M and N/P = 300
    (512, 1024, 2048, 8),          # 128 x 64 tiles, whole tiles
    (256, 64 * 8, 256 * 8, 8),     # 128 x 64 tiles, K/P = 64 (one K step)
    (200, 512, 260 * 4, 4),        # 128 x 64 tiles, two M tiles, ragged M and N/P = 260
    (100, 256, 2200 * 8, 8),       # 128 x 128 tiles (144, more than half the CUs), N/P = 2200
    (130, 512, 1100 * 8, 8),       # 128 x 128 tiles, two M tiles, ragged M and N/P = 1100
    (1024, 64 * 8, 1024 * 8, 8),   # column: 256 x 128 tiles (128-row tiles would not fit one pass)
    (520, 1024, 2048, 4),          # row partials: 256 x 128 tiles, ragged M; column: 128 x 64
    (1100, 1024, 264 * 16, 16),    # 256 x 256 tile kernel (160 tiles), ragged M and N/P = 264
    (40, 24, 42, 3),               # skinny with K/P = 8 (K tail)
    (257, 72 * 2, 130, 2),         # generic (K/P = 72 is not a multiple of 64)
]


@pytest.mark.parametrize("case", range(len(ALIGNED)))
def test_kernel_paths_bitwise(case):
    M, K, N, P = ALIGNED[case]
    print(f"case M={M} K={K} N={N} P={P}", flush=True)
    Xd, Wd, X64, Wio = _inputs_int(500 + case, M, K, N, torch.bfloat16)
    _run_all_modes(Xd, Wd, X64, Wio, M, K, N, P, torch.bfloat16)


# The decode kernel pipelines K in stages (column and partial forms: three
# stages of 256 columns; fused fold: five).  In the last stages fewer later
# stages exist, so the waits there differ; these shapes give every count of
# stages from 1 to 12 per workgroup (K per shard 256*s, P shards walked by
# the fused form), with and without a ragged last stage, and a fused
# workgroup whose second 16-column block is partly past N.
STAGES = [(M, (256 * s + tail) * P, 48, P)
          for M in (16, 7, 1) for P in (1, 2) for s in (1, 2, 3, 4, 5, 6) for tail in (0, 8)
          if not (M != 16 and tail)]


@pytest.mark.parametrize("case", range(len(STAGES)))
def test_decode_stage_counts_bitwise(case):
    M, K, N, P = STAGES[case]
    print(f"case M={M} K={K} N={N} P={P}", flush=True)
    Xd, Wd, X64, Wio = _inputs_int(900 + case, M, K, N, torch.bfloat16)
    _run_all_modes(Xd, Wd, X64, Wio, M, K, N, P, torch.bfloat16)


def test_strided_views_bitwise():
    # Leading dims larger than the row width (views into bigger buffers).
    M, K, N, P = 70, 256, 128, 4
    Xb = synth.small_ints(7, (M, K + 8))
    Wb = synth.small_ints(8, (N, K + 24))
    Xd = bf16_dev(synth.to_bf16_bits(Xb))[:, :K]
    Wd = bf16_dev(synth.to_bf16_bits(Wb))[:, :K]
    X64, Wio = Xb[:, :K].astype(np.float64), Wb[:, :K].T.astype(np.float64)
    Ybuf = torch.full((M, N + 16), float("nan"), dtype=torch.bfloat16, device=DEV)
    Y = Ybuf[:, :N]
    tl.tp_linear_column(Xd, Wd, Y, P)
    assert np.array_equal(bits(Y), expected_bits(oracle.column_parallel_linear(X64, Wio, P),
                                                 torch.bfloat16))
    assert torch.isnan(Ybuf[:, N:].float()).all(), "wrote outside the view"
    Ybuf.fill_(float("nan"))
    tl.tp_linear_row(Xd, Wd, Y, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P))
    assert np.array_equal(bits(Y), expected_bits(oracle.row_parallel_linear(X64, Wio, P),
                                                 torch.bfloat16))
    assert torch.isnan(Ybuf[:, N:].float()).all()


# ---------------------------------------------------------------------------
# Shard fold: bit-exact against the oracle's fp32 left fold + RNE.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P,M,N", [(8, 64, 512), (8, 37, 1000), (1, 5, 8), (3, 7, 5),
                                   (8, 256, 4096), (64, 3, 24), (13, 9, 16)])
def test_shard_reduce_bitexact(P, M, N):
    parts = synth.normal_f32(P * 1000 + M, (P, M, N)) * np.float32(4.0)
    want32 = oracle.fold_f32(parts)
    pd = f32_dev(parts)
    for dtype in (torch.bfloat16, torch.float32):
        Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
        tl.tp_shard_reduce(pd, Y, P)
        want = oracle.round_bf16(want32) if dtype == torch.bfloat16 else want32.view(np.uint32)
        assert np.array_equal(bits(Y), want)
        if M % P == 0:
            # scatter into separate slots with a gap between slices
            s = M // P
            gap = 3 * N + 8
            buf = torch.full((P * gap * s + 64,), float("nan"), dtype=dtype, device=DEV)
            tl.tp_shard_reduce(pd, buf[: s * N].view(s, N), P, scatter=1, y_slice_stride=s * gap)
            for j in range(P):
                got = buf[j * s * gap: j * s * gap + s * N].view(s, N)
                assert np.array_equal(bits(got), want[j * s:(j + 1) * s])


def test_shard_reduce_order_cases():
    # The hand-derived fold cases (tests/golden) on the device.
    import json, os
    with open(os.path.join(os.path.dirname(__file__), "golden", "fold_f32_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        P = len(c["parts"])
        parts = np.array([int(h, 16) for h in c["parts"]], dtype=np.uint32).view(np.float32)
        pd = f32_dev(np.repeat(parts.reshape(P, 1, 1), 8, axis=2))
        Y = torch.empty((1, 8), dtype=torch.float32, device=DEV)
        tl.tp_shard_reduce(pd, Y, P)
        assert np.all(bits(Y) == np.uint32(int(c["fold"], 16))), c["why"]


# ---------------------------------------------------------------------------
# Worked example ("模型并行", "Tensor-parallel 线性层"): fp32, P = 4.
# ---------------------------------------------------------------------------

def test_worked_example_fp32():
    torch.manual_seed(0)
    x, w = torch.randn(3, 8), torch.randn(8, 12)
    dense = x @ w
    X64, Wio = oracle.widen_f32(x.numpy()), oracle.widen_f32(w.numpy())
    ref = oracle.dense(X64, Wio)
    Xd = x.to(DEV)
    Wd = w.t().contiguous().to(DEV)  # [N, K] storage
    Y = torch.empty((3, 12), device=DEV)
    tl.tp_linear_column(Xd, Wd, Y, 4)
    assert Y.shape == (3, 12)
    assert oracle.rel_l2(to_f64(Y), ref) <= 1e-5
    torch.testing.assert_close(Y.cpu(), dense)
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
        Y = torch.empty((3, 12), device=DEV)
        tl.tp_linear_row(Xd, Wd, Y, 4, mode, workspace(mode, 3, 12, 4))
        assert oracle.rel_l2(to_f64(Y), ref) <= 1e-5
        torch.testing.assert_close(Y.cpu(), dense)
    Yp = torch.empty((4, 3, 12), device=DEV)
    tl.tp_linear_row(Xd, Wd, Yp, 4, tl.TP_ROW_PARTIAL)
    for i, pi in enumerate(oracle.row_partials(X64, Wio, 4)):
        assert oracle.rel_l2(to_f64(Yp[i]), pi) <= 1e-5


def test_worked_example_numpy_seeds():
    X = synth.normal_f32(synth.seed_for(1, 0, 0), (3, 8))
    W = synth.normal_f32(synth.seed_for(1, 0, 1), (12, 8))
    X64, Wio = oracle.widen_f32(X), oracle.widen_f32(W).T
    ref = oracle.dense(X64, Wio)
    Y = torch.empty((3, 12), device=DEV)
    tl.tp_linear_column(f32_dev(X), f32_dev(W), Y, 4)
    assert oracle.rel_l2(to_f64(Y), ref) <= 1e-5
    tl.tp_linear_row(f32_dev(X), f32_dev(W), Y, 4, tl.TP_ROW_SUM,
                     workspace(tl.TP_ROW_SUM, 3, 12, 4))
    assert oracle.rel_l2(to_f64(Y), ref) <= 1e-5


# ---------------------------------------------------------------------------
# Workload shapes with reduced M (full N, K, P), N(0,1) x N(0,0.02^2) bf16.
# ---------------------------------------------------------------------------

REDUCED = [
    # (workload, form, M, K, N, P)
    (2, "column", 300, 4096, 28672, 8),
    (2, "row", 300, 14336, 4096, 8),
    (3, "column", 264, 8192, 10240, 8),
    (3, "row", 264, 8192, 8192, 8),
    (4, "column", 16, 8192, 28672, 8),
    (4, "row_fused", 16, 28672, 8192, 8),
    (5, "row_scatter", 264, 28672, 8192, 8),
]


@pytest.mark.parametrize("case", range(len(REDUCED)))
def test_workload_shapes_reduced_m(case):
    cfg, form, M, K, N, P = REDUCED[case]
    print(f"workload {cfg} {form} M={M} K={K} N={N} P={P}", flush=True)
    g = 0
    Xb = synth.normal_bf16(synth.seed_for(cfg, g, 0) + 7, (M, K), synth.SIGMA_X)
    Wb = synth.normal_bf16(synth.seed_for(cfg, g, 1) + 7, (N, K), synth.SIGMA_W)
    Xd, Wd = bf16_dev(Xb), bf16_dev(Wb)
    X64, Wio = oracle.widen_bf16(Xb), oracle.widen_bf16(Wb).T
    tol = bf16_tol(K)
    if form == "column":
        ref = oracle.column_parallel_linear(X64, Wio, P)
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_column(Xd, Wd, Y, P)
        got = to_f64(Y)
    else:
        parts = oracle.row_partials(X64, Wio, P)
        ref = oracle.fold_f64(parts)
        mode = {"row": tl.TP_ROW_SUM, "row_fused": tl.TP_ROW_FUSED,
                "row_scatter": tl.TP_ROW_SCATTER}[form]
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_row(Xd, Wd, Y, P, mode, workspace(mode, M, N, P))
        got = to_f64(Y)
        # partials in fp32: each within the fp32 bar of its exact value
        Yp = torch.empty((P, M, N), dtype=torch.float32, device=DEV)
        tl.tp_linear_row(Xd, Wd, Yp, P, tl.TP_ROW_PARTIAL)
        for i, pi in enumerate(parts):
            assert oracle.rel_l2(to_f64(Yp[i]), pi) <= 1e-5, f"partial {i}"
    r, a = oracle.rel_l2(got, ref), oracle.max_abs(got, ref)
    print(f"rel_l2={r:.3e} max_abs={a:.3e} bar={tol:.3e}", flush=True)
    assert r <= 1e-2
    assert a <= tol
