"""The row GEMM with the shard fold in registers (TP_ROW_FUSED for prefill
shapes): bitwise equal to the unfused sequence (fp32 partials + ascending
fold, TP_ROW_SUM) on N(0,1) x N(0, 0.02^2) data at the workload shapes with
reduced M, with and without the row bias, ragged M and N tiles, P = 1, and
against the oracle on sampled rows.  These shapes have fewer tiles than the
library takes the fold in registers for by itself, so every test here runs
with TPLINEAR_ROW_FOLD=gemm, which sends every shape the kernel takes to it."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import DEV, bits, to_f64, workspace, bf16_tol, row_fold

pytestmark = pytest.mark.gpu


@pytest.fixture(autouse=True)
def _fold_in_gemm():
    with row_fold("gemm"):
        yield

SHAPES = [
    # (M, K, N, P, bias)
    (512, 16384, 4096, 8, False),   # K/P = 2048, the longest shard K taken at any size
    (4096, 28672, 4096, 8, False),  # K/P = 3584 with a 4096 x 4096 output
    (264, 8192, 8192, 8, True),     # Llama-70B O, K/P = 1024, ragged M tile
    (300, 1024, 1000, 8, True),     # ragged N tile (1000 = 7 x 128 + 104)
    (256, 256, 136, 2, False),
    (320, 512, 384, 1, True),       # P = 1: the plain GEMM
    (256, 192, 256, 3, True),       # P = 3, K/P = 64: one K step per shard
    (300, 4096, 200, 64, False),    # P = 64 (the most shards), K/P = 64, ragged M and N
]


def _rand(gen, shape, s=1.0):
    return (torch.randn(shape, generator=gen, device=DEV) * s).to(torch.bfloat16)


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_fused_fold_equals_partials_and_fold(case):
    M, K, N, P, with_bias = SHAPES[case]
    print(f"rowfold M={M} K={K} N={N} P={P} bias={with_bias}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(100 + case)
    X, W = _rand(gen, (M, K)), _rand(gen, (N, K), 0.02)
    b = _rand(gen, (N,), 0.02) if with_bias else None
    Ys = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Yf = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row_ex(X, W, Ys, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P), bias=b)
    # the fused form needs no workspace contents; give it a poisoned one
    ws = workspace(tl.TP_ROW_FUSED, M, N, P, zero=False)
    ws.fill_(0xFF)
    tl.tp_linear_row_ex(X, W, Yf, P, tl.TP_ROW_FUSED, ws, bias=b)
    assert np.array_equal(bits(Ys), bits(Yf))
    assert bool(torch.all(ws == 0xFF)), "the fused fold touched the workspace"
    # sampled rows against the fp64 oracle
    rows = [0, M // 2, M - 1]
    X64 = to_f64(X[rows])
    Wio = np.ascontiguousarray(to_f64(W).T)
    ref = oracle.row_parallel_linear(X64, Wio, P)
    if with_bias:
        ref = ref + to_f64(b)[None, :]
    got = to_f64(Yf[rows])
    assert oracle.rel_l2(got, ref) <= 1e-2
    assert oracle.max_abs(got, ref) <= bf16_tol(K, 1.0, 0.02)


def test_fused_fold_repeat_and_strided_output():
    # a strided output view with guard columns, called twice
    M, K, N, P = 300, 2048, 520, 4
    gen = torch.Generator(device=DEV)
    gen.manual_seed(7)
    X, W = _rand(gen, (M, K)), _rand(gen, (N, K), 0.02)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row(X, W, ref, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P))
    buf = torch.full((M, N + 24), -7.0, dtype=torch.bfloat16, device=DEV)
    view = buf[:, 8:8 + N]
    for _ in range(2):
        tl.tp_linear_row(X, W, view, P, tl.TP_ROW_FUSED, workspace(tl.TP_ROW_FUSED, M, N, P))
        torch.cuda.synchronize()
        assert np.array_equal(bits(view), bits(ref))
        assert bool(torch.all(buf[:, :8] == -7.0)) and bool(torch.all(buf[:, 8 + N:] == -7.0))


@pytest.mark.parametrize("M,K,N,P,slices", [
    (2048, 8192, 1024, 8, False),
    (2048, 8192, 1024, 8, True),
    # P = 1 with a slice allocation: one slice, the whole (ragged) output,
    # written through the slice table (a regression case: this shape once
    # took the path that writes through Y, which is NULL with y_slices)
    (320, 512, 384, 1, True),
    (320, 512, 384, 1, False),
])
def test_fused_reduce_scatter(M, K, N, P, slices):
    # M/P = 256-row token slices (or one slice): the reduce-scatter runs as
    # the fused fold; its slices equal the rows of TP_ROW_SUM bit for bit.
    print(f"fused reduce-scatter M={M} K={K} N={N} P={P} slices={slices}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(11)
    X, W = _rand(gen, (M, K)), _rand(gen, (N, K), 0.02)
    b = _rand(gen, (N,), 0.02)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row_ex(X, W, ref, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P), bias=b)
    s = M // P
    ws = workspace(tl.TP_ROW_SCATTER, M, N, P, zero=False)
    ws.fill_(0xFF)
    if slices:
        out = [torch.full((s, N + 8), float("nan"), dtype=torch.bfloat16, device=DEV)[:, :N]
               for _ in range(P)]
        tl.tp_linear_row_ex(X, W, None, P, tl.TP_ROW_SCATTER, ws, bias=b, y_slices=out)
    else:
        Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_row_ex(X, W, Y, P, tl.TP_ROW_SCATTER, ws, bias=b)
        out = [Y[j * s:(j + 1) * s] for j in range(P)]
    for j in range(P):
        assert np.array_equal(bits(out[j]), bits(ref[j * s:(j + 1) * s])), j
    assert bool(torch.all(ws == 0xFF)), "the fused reduce-scatter touched the workspace"
