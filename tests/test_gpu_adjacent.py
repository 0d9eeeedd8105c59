"""GPU parity of the steps next to the Linear, through the C ABI, against the
CPU oracle on the same seeded inputs:

  * column bias (Shard(0)) and row bias (Partial(), once after the fold):
    bit for bit on integer-valued inputs on every kernel path and row mode,
    and on the hand-derived fp32 fold+bias cases;
  * the gated unit of a fused gate+up column layer: on integer-valued inputs
    the gate and up products are exact, so the only error left is the fp32
    silu and the final bf16 rounding (|err| <= 2^-8 |ref|); at the Llama-8B
    MLP shape (reduced M) with N(0,1) x N(0, 0.02^2) inputs, rel L2 <= 1e-2
    and the per-element bound of the bf16 bar carried through silu(g) * u;
  * token slices in separate allocations: the column layer reading them and
    the reduce-scatter writing them, bit for bit against the oracle
    (integers) and against the contiguous layout (random data);
  * the feature-sharded embedding: bit-exact copies, both table layouts and
    both output layouts, zero rows and the flag for ids outside [0, V).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import (DEV, FOLD_POLICIES, bf16_dev, f32_dev, to_f64, bits, expected_bits, row_fold,
                      workspace, bf16_tol)

pytestmark = pytest.mark.gpu

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _dev(a, dtype):
    a = np.ascontiguousarray(a, dtype=np.float32)
    return bf16_dev(synth.to_bf16_bits(a)) if dtype == torch.bfloat16 else f32_dev(a)


def _ints(seed, shape, lo=-2, hi=2):
    return synth.small_ints(seed, shape, lo, hi)


# ---------------------------------------------------------------------------
# Column bias, bitwise on integer inputs.
# (M, K, N, P, dtype): skinny, tile (bias_shard a multiple of 8), tile-shaped
# but a bias offset that sends it to the generic kernel, fp32 generic.
# ---------------------------------------------------------------------------

BIAS_COL = [
    (7, 512, 3 * 48, 3, torch.bfloat16),     # skinny
    (40, 256, 2 * 16, 2, torch.bfloat16),    # skinny, M in (32, 48]
    (300, 128, 2 * 264, 2, torch.bfloat16),  # tile, ragged M and N/P = 264
    (512, 256, 4 * 256, 4, torch.bfloat16),  # tile, whole tiles
    (300, 128, 2 * 260, 2, torch.bfloat16),  # N/P = 260: bias offset not a multiple of 8 -> generic
    (5, 12, 3 * 7, 3, torch.float32),        # fp32 generic
]


@pytest.mark.parametrize("case", range(len(BIAS_COL)))
def test_column_bias_bitwise(case):
    M, K, N, P, dtype = BIAS_COL[case]
    print(f"column bias M={M} K={K} N={N} P={P} {dtype}", flush=True)
    X, W = _ints(900 + case, (M, K)), _ints(901 + case, (N, K))
    b = _ints(902 + case, (N,), -8, 8)
    Xd, Wd, bd = _dev(X, dtype), _dev(W, dtype), _dev(b, dtype)
    ref = oracle.column_parallel_linear_bias(X.astype(np.float64), W.T.astype(np.float64),
                                             b.astype(np.float64), P)
    Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column_ex(Xd, Wd, Y, P, bias=bd)
    assert np.array_equal(bits(Y), expected_bits(ref, dtype)), "concat"
    Ys = torch.full((P, M, N // P), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column_ex(Xd, Wd, Ys, P, y_mode=tl.TP_Y_SHARDS, bias=bd)
    s = N // P
    for i in range(P):
        assert np.array_equal(bits(Ys[i]), expected_bits(ref[:, i * s:(i + 1) * s], dtype)), i


def test_column_ex_without_options_equals_column():
    # No bias, no activation, X given: the same kernel as tp_linear_column.
    M, K, N, P = 300, 256, 2 * 264, 2
    X = synth.normal_bf16(11, (M, K))
    W = synth.normal_bf16(12, (N, K), 0.02)
    Xd, Wd = bf16_dev(X), bf16_dev(W)
    Y0 = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Y1 = torch.empty_like(Y0)
    tl.tp_linear_column(Xd, Wd, Y0, P)
    tl.tp_linear_column_ex(Xd, Wd, Y1, P)
    assert torch.equal(Y0.view(torch.int16), Y1.view(torch.int16))


# ---------------------------------------------------------------------------
# Row bias: every row mode, bitwise on integer inputs; the fold+bias golden
# cases on the device; fused == sum and partial + fold == sum on random data.
# ---------------------------------------------------------------------------

BIAS_ROW = [
    (16, 3 * 512, 48, 3, torch.bfloat16),    # fused decode kernel (bias after the fold)
    (24, 3 * 256, 48, 3, torch.bfloat16),    # fused decode, two m-blocks; scatter
    (8, 2 * 256, 40, 2, torch.bfloat16),     # fused decode, ragged 32-column block
    (256, 2 * 128, 264, 2, torch.bfloat16),  # tile partials + fold
    (12, 4 * 3, 9, 4, torch.float32),        # fp32 generic + fold (scalar path)
]


@pytest.mark.parametrize("case", range(len(BIAS_ROW)))
def test_row_bias_bitwise(case):
    M, K, N, P, dtype = BIAS_ROW[case]
    print(f"row bias M={M} K={K} N={N} P={P} {dtype}", flush=True)
    X, W = _ints(920 + case, (M, K)), _ints(921 + case, (N, K))
    b = _ints(922 + case, (N,), -8, 8)
    Xd, Wd, bd = _dev(X, dtype), _dev(W, dtype), _dev(b, dtype)
    X64, Wio = X.astype(np.float64), W.T.astype(np.float64)
    ref = oracle.row_parallel_linear_bias(X64, Wio, b.astype(np.float64), P)
    for policy in FOLD_POLICIES:
        with row_fold(policy):
            for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
                Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
                tl.tp_linear_row_ex(Xd, Wd, Y, P, mode, workspace(mode, M, N, P), bias=bd)
                assert np.array_equal(bits(Y), expected_bits(ref, dtype)), f"mode {mode} {policy}"
            if M % P == 0:
                Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
                tl.tp_linear_row_ex(Xd, Wd, Y, P, tl.TP_ROW_SCATTER,
                                    workspace(tl.TP_ROW_SCATTER, M, N, P), bias=bd)
                assert np.array_equal(bits(Y), expected_bits(ref, dtype)), f"scatter {policy}"
    # partials + the fold with bias
    Yp = torch.empty((P, M, N), dtype=torch.float32, device=DEV)
    tl.tp_linear_row(Xd, Wd, Yp, P, tl.TP_ROW_PARTIAL)
    Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
    tl.tp_shard_reduce_ex(Yp, Y, P, bias=bd)
    assert np.array_equal(bits(Y), expected_bits(ref, dtype)), "partials + fold"


def _f32(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


def test_fold_bias_golden_cases_on_device():
    cases = json.load(open(os.path.join(GOLDEN, "fold_bias_f32_cases.json")))["cases"]
    for c in cases:
        parts = np.array([_f32(h) for h in c["parts"]], dtype=np.float32)
        P = parts.size
        # fill a [P, 2, 8] block with the case (every element the same), fp32 out
        p = torch.from_numpy(np.broadcast_to(parts[:, None, None], (P, 2, 8)).copy()).to(DEV)
        b = torch.full((8,), float(_f32(c["bias"])), dtype=torch.float32, device=DEV)
        Y = torch.empty((2, 8), dtype=torch.float32, device=DEV)
        tl.tp_shard_reduce_ex(p, Y, P, bias=b)
        got = bits(Y)
        assert np.all(got == int(c["out"], 16)), c["why"]


@pytest.mark.parametrize("P", [1, 3, 8])
def test_row_bias_fused_equals_sum_random(P):
    M, K, N = 16, 512 * P, 1000
    X = synth.normal_bf16(31 + P, (M, K))
    W = synth.normal_bf16(32 + P, (N, K), 0.02)
    b = synth.normal_bf16(33 + P, (N,), 0.5)
    Xd, Wd, bd = bf16_dev(X), bf16_dev(W), bf16_dev(b)
    Ys = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    Yf = torch.empty_like(Ys)
    tl.tp_linear_row_ex(Xd, Wd, Ys, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P), bias=bd)
    ws = workspace(tl.TP_ROW_FUSED, M, N, P)
    for policy in FOLD_POLICIES:
        with row_fold(policy):
            tl.tp_linear_row_ex(Xd, Wd, Yf, P, tl.TP_ROW_FUSED, ws, bias=bd)
        assert torch.equal(Ys.view(torch.int16), Yf.view(torch.int16)), policy
    # partials, then the fold with the bias: the same bits again
    Yp = torch.empty((P, M, N), dtype=torch.float32, device=DEV)
    tl.tp_linear_row(Xd, Wd, Yp, P, tl.TP_ROW_PARTIAL)
    Y2 = torch.empty_like(Ys)
    tl.tp_shard_reduce_ex(Yp, Y2, P, bias=bd)
    assert torch.equal(Y2.view(torch.int16), Yf.view(torch.int16))


@pytest.mark.parametrize("N", [1000, 999])
@pytest.mark.parametrize("out", ["bf16", "f32"])
def test_fold_bias_synthetic_bitwise(N, out):
    # Synthetic fp32 partials (seeded, not produced by the library), P = 8:
    # the fold with the bias, plain and scattered into slice allocations,
    # equals the oracle's fp32 left fold + bias (+ its RNE) bit for bit.
    # N = 999 takes the scalar fold.
    P, M = 8, 40
    parts = synth.normal_f32(71, (P, M, N))
    dtype = torch.bfloat16 if out == "bf16" else torch.float32
    if dtype == torch.bfloat16:
        bb = synth.normal_bf16(72, (N,), 0.3)
        b32, bd = oracle.widen_bf16(bb).astype(np.float32), bf16_dev(bb)
    else:
        b32 = synth.normal_f32(72, (N,), 0.3)
        bd = f32_dev(b32)
    fold = oracle.fold_f32(parts, b32)
    ref = oracle.round_bf16(fold) if dtype == torch.bfloat16 else fold.view(np.uint32)
    pd = f32_dev(parts)
    Y = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
    tl.tp_shard_reduce_ex(pd, Y, P, bias=bd)
    assert np.array_equal(bits(Y), ref)
    s = M // P
    slices = [torch.full((s, N + 4), float("nan"), dtype=dtype, device=DEV)[:, :N] for _ in range(P)]
    tl.tp_shard_reduce_ex(pd, None, P, scatter=1, bias=bd, y_slices=slices)
    for j in range(P):
        assert np.array_equal(bits(slices[j]), ref[j * s:(j + 1) * s]), j


# ---------------------------------------------------------------------------
# The gated unit.
# ---------------------------------------------------------------------------

SWIGLU = [
    # (M, K, I, P, dtype, with_bias)
    (9, 256, 2 * 24, 2, torch.bfloat16, True),     # skinny (16 gate + 16 up rows per workgroup)
    (40, 256, 2 * 24, 2, torch.bfloat16, False),   # skinny, two m-blocks
    (300, 128, 2 * 136, 2, torch.bfloat16, True),  # narrow 128-row tiles, ragged M, I/P = 136
    (512, 128, 4 * 128, 4, torch.bfloat16, False),  # narrow 128-row tiles, whole tiles
    (1024, 128, 8 * 512, 8, torch.bfloat16, True),  # narrow 256-row tiles
    (1100, 128, 16 * 256, 16, torch.bfloat16, True),  # 256 x 256 tile kernel (160 tiles), ragged M
    (300, 128, 2 * 132, 2, torch.bfloat16, True),  # I/P = 132: up offset not a multiple of 8 -> generic
    (5, 10, 2 * 3, 2, torch.float32, True),        # fp32 generic
]


def test_swiglu_kernels_agree_on_rows():
    """The gated unit on the 256 x 256 tile kernel and on both narrow tile
    shapes: the first rows of a longer launch equal a shorter launch bit for
    bit (an output row depends only on its X row, and these kernels add K in
    the same order), on N(0,1) x N(0, 0.02^2) data with the bias."""
    P, On, K = 16, 256, 256
    N = 2 * On * P
    X = bf16_dev(synth.normal_bf16(71, (1100, K)))
    W = bf16_dev(synth.normal_bf16(72, (N, K), 0.02))
    b = bf16_dev(synth.normal_bf16(73, (N,), 0.02))
    outs = {}
    for M in (1100, 600, 300):   # 160 tiles of 256 x 256; narrow 256-row; narrow 128-row
        print(f"swiglu rows M={M}", flush=True)
        Y = torch.full((M, On * P), float("nan"), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_column_ex(X[:M], W, Y, P, bias=b, act=tl.TP_ACT_SWIGLU)
        outs[M] = bits(Y)
    assert np.array_equal(outs[600], outs[1100][:600])
    assert np.array_equal(outs[300], outs[1100][:300])


@pytest.mark.parametrize("case", range(len(SWIGLU)))
def test_swiglu_integer_inputs(case):
    M, K, I, P, dtype, with_bias = SWIGLU[case]
    print(f"swiglu M={M} K={K} I={I} P={P} {dtype} bias={with_bias}", flush=True)
    N = 2 * I
    X, W = _ints(940 + case, (M, K)), _ints(941 + case, (N, K))
    b = _ints(942 + case, (N,), -3, 3) if with_bias else None
    Xd, Wd = _dev(X, dtype), _dev(W, dtype)
    bd = _dev(b, dtype) if with_bias else None
    ref = oracle.column_parallel_swiglu(X.astype(np.float64), W.T.astype(np.float64),
                                        None if b is None else b.astype(np.float64), P)
    Y = torch.full((M, I), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column_ex(Xd, Wd, Y, P, bias=bd, act=tl.TP_ACT_SWIGLU)
    got = to_f64(Y)
    # gate and up are exact integers: only the fp32 silu and one rounding
    # to the output type remain.
    # fp32: the fast exponential is exp2(g log2 e); the rounding of g log2 e
    # gives a relative error of about |g| 2^-24 ln 2 log2 e, under 2^-14 for
    # the |g| <= 64 of these inputs.
    rel = 2.0 ** -8 if dtype == torch.bfloat16 else 2.0 ** -14
    err = np.abs(got - ref)
    assert np.all(np.isfinite(got))
    assert np.all(err <= rel * np.abs(ref) + 1e-30), float(np.max(err - rel * np.abs(ref)))
    Ys = torch.full((P, M, I // P), float("nan"), dtype=dtype, device=DEV)
    tl.tp_linear_column_ex(Xd, Wd, Ys, P, y_mode=tl.TP_Y_SHARDS, bias=bd, act=tl.TP_ACT_SWIGLU)
    s = I // P
    for i in range(P):
        assert np.array_equal(bits(Ys[i]), bits(Y[:, i * s:(i + 1) * s])), i


def _swiglu_bound(G, U, K, sw):
    """Per-element bar for silu(g) * u: the bf16 bar of each product,
    t = 2e-2 sqrt(K) sx sw, carried through the unit to first order,
    |d/dg| t + |d/du| t, plus one bf16 rounding of the output (2^-8 |h|)."""
    t = bf16_tol(K, synth.SIGMA_X, sw)
    sig = 1.0 / (1.0 + np.exp(-G))
    dsilu = sig * (1.0 + G * (1.0 - sig))
    h = G * sig * U
    return t * (np.abs(dsilu * U) + np.abs(G * sig)) + 2.0 ** -8 * np.abs(h)


def test_swiglu_llama8b_mlp_shape_reduced_m():
    # fc1 gate+up of the Llama-8B MLP shard: K = 4096, I = 14336, P = 8, with
    # a column bias; M reduced to 264 rows (two M tiles, the second ragged).
    M, K, I, P = 264, 4096, 14336, 8
    X = synth.normal_bf16(synth.seed_for(2, 0, 0), (M, K), synth.SIGMA_X)
    W = synth.normal_bf16(synth.seed_for(2, 0, 1), (2 * I, K), synth.SIGMA_W)
    b = synth.normal_bf16(synth.seed_for(2, 0, 2), (2 * I,), synth.SIGMA_W)
    Xd, Wd, bd = bf16_dev(X), bf16_dev(W), bf16_dev(b)
    Y = torch.empty((M, I), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_column_ex(Xd, Wd, Y, P, bias=bd, act=tl.TP_ACT_SWIGLU)
    got = to_f64(Y)
    G, U = oracle.column_parallel_gate_up(oracle.widen_bf16(X), oracle.widen_bf16(W).T,
                                          oracle.widen_bf16(b), P)
    ref = oracle.swiglu(G, U)
    r = oracle.rel_l2(got, ref)
    bound = _swiglu_bound(G, U, K, synth.SIGMA_W)
    worst = float(np.max(np.abs(got - ref) / bound))
    print(f"swiglu fc1: rel_l2={r:.3e} worst err/bound={worst:.3f}", flush=True)
    assert r <= 1e-2
    assert worst <= 1.0


# ---------------------------------------------------------------------------
# Token slices in separate allocations.
# ---------------------------------------------------------------------------

GATHER = [
    # (M, K, N, P, act, bias): 256-row slices reach the tile kernel; others generic
    (1024, 256, 4 * 256, 4, tl.TP_ACT_NONE, False),
    (1024, 256, 4 * 272, 4, tl.TP_ACT_SWIGLU, True),
    (512, 128, 2 * 264, 2, tl.TP_ACT_NONE, True),
    (24, 64, 4 * 8, 4, tl.TP_ACT_NONE, False),      # 6-row slices: generic
    (600, 64, 3 * 40, 3, tl.TP_ACT_SWIGLU, False),  # 200-row slices: generic
]


@pytest.mark.parametrize("case", range(len(GATHER)))
def test_gathered_column_bitwise(case):
    M, K, N, P, act, with_bias = GATHER[case]
    print(f"gathered M={M} K={K} N={N} P={P} act={act} bias={with_bias}", flush=True)
    X, W = _ints(960 + case, (M, K)), _ints(961 + case, (N, K))
    b = _ints(962 + case, (N,), -4, 4) if with_bias else None
    s = M // P
    # each slice in its own allocation, with a row stride wider than K
    slices = []
    for j in range(P):
        buf = torch.full((s, K + 8), float("nan"), dtype=torch.bfloat16, device=DEV)
        buf[:, :K] = _dev(X[j * s:(j + 1) * s], torch.bfloat16)
        slices.append(buf[:, :K])
    Wd = _dev(W, torch.bfloat16)
    bd = _dev(b, torch.bfloat16) if with_bias else None
    On = N // P // (2 if act == tl.TP_ACT_SWIGLU else 1)
    Y = torch.full((M, On * P), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_column_ex(None, Wd, Y, P, bias=bd, act=act, x_slices=slices)
    # the same product on the contiguous X, and the oracle on the gathered slices
    Xc = _dev(X, torch.bfloat16)
    Yc = torch.empty_like(Y)
    tl.tp_linear_column_ex(Xc, Wd, Yc, P, bias=bd, act=act)
    X64 = [X[j * s:(j + 1) * s].astype(np.float64) for j in range(P)]
    if act == tl.TP_ACT_NONE:
        ref = oracle.column_parallel_linear_gathered(X64, W.T.astype(np.float64), P)
        if b is not None:
            ref = ref + np.concatenate([b[i * (N // P):(i + 1) * (N // P)] for i in range(P)])[None, :]
        assert np.array_equal(bits(Y), expected_bits(ref, torch.bfloat16))
        assert np.array_equal(bits(Yc), bits(Y))
    else:
        ref = oracle.column_parallel_swiglu(oracle.all_gather_rows(X64), W.T.astype(np.float64),
                                            None if b is None else b.astype(np.float64), P)
        got = to_f64(Y)
        assert np.all(np.abs(got - ref) <= 2.0 ** -8 * np.abs(ref) + 1e-30)
        # same kernel on both layouts when the slices are whole tiles
        if s % 256 == 0:
            assert np.array_equal(bits(Yc), bits(Y))


def test_reduce_scatter_to_slices_then_gathered_column():
    # The sequence-parallel round trip at the workload's K and N with reduced
    # M: row GEMM, reduce-scatter into P separate slice allocations, the next
    # column layer reading the slices in place.  Bitwise equal to the
    # contiguous layout, and the slices equal the oracle's fold bit for bit.
    M, K, N, N3, P = 2048, 28672, 8192, 1024, 8
    g = torch.Generator(device=DEV)
    g.manual_seed(5)
    X = (torch.randn((M, K), generator=g, device=DEV)).to(torch.bfloat16)
    W = (torch.randn((N, K), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    W3 = (torch.randn((N3, N), generator=g, device=DEV) * 0.02).to(torch.bfloat16)
    ws = workspace(tl.TP_ROW_SCATTER, M, N, P, zero=False)
    s = M // P
    slices = [torch.empty((s, N), dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    tl.tp_linear_row_ex(X, W, None, P, tl.TP_ROW_SCATTER, ws, y_slices=slices)
    Yc = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row(X, W, Yc, P, tl.TP_ROW_SCATTER, ws)
    for j in range(P):
        assert torch.equal(slices[j].view(torch.int16), Yc[j * s:(j + 1) * s].view(torch.int16)), j
    # sampled token rows against the oracle (each output row depends on its
    # own input row and all of W)
    rows = [0, s + 3, M - 1]
    X64 = to_f64(X[rows])
    Wio = np.ascontiguousarray(to_f64(W).T)
    ref = oracle.row_parallel_linear(X64, Wio, P)
    got = np.stack([to_f64(slices[r // s][r % s:r % s + 1])[0] for r in rows])
    assert oracle.rel_l2(got, ref) <= 1e-2
    assert oracle.max_abs(got, ref) <= bf16_tol(K, 1.0, 0.02)
    del Wio
    Y3 = torch.empty((M, N3), dtype=torch.bfloat16, device=DEV)
    Y3c = torch.empty_like(Y3)
    tl.tp_linear_column_ex(None, W3, Y3, P, x_slices=slices)
    tl.tp_linear_column(Yc, W3, Y3c, P)
    assert torch.equal(Y3.view(torch.int16), Y3c.view(torch.int16))


# ---------------------------------------------------------------------------
# Embedding.
# ---------------------------------------------------------------------------

EMB = [
    # (V, D, T, P, dtype): 16-byte pieces reach the vector kernel; others scalar
    (1000, 512, 300, 8, torch.bfloat16),
    (77, 64, 50, 4, torch.float32),
    (50, 12, 33, 4, torch.bfloat16),      # 3 features per shard: scalar path
    (90, 384, 13, 3, torch.bfloat16),     # 39 pieces: a partial group of 8 per wavefront
    (128256, 4096, 64, 8, torch.bfloat16),  # Llama-8B vocabulary and width
]


def _table(seed, V, D, dtype):
    if dtype == torch.bfloat16:
        bits_ = synth.normal_bf16(seed, (V, D))
        return bits_, bf16_dev(bits_)
    a = synth.normal_f32(seed, (V, D))
    return a.view(np.uint32), f32_dev(a)


@pytest.mark.parametrize("case", range(len(EMB)))
def test_embedding_bitwise(case):
    V, D, T, P, dtype = EMB[case]
    print(f"embedding V={V} D={D} T={T} P={P} {dtype}", flush=True)
    Eb, Ed = _table(980 + case, V, D, dtype)
    ids = np.random.default_rng(case).integers(0, V, size=T)
    idd = torch.from_numpy(ids.astype(np.int64)).to(DEV)
    ref = oracle.embedding_parallel(ids, Eb, P)            # bit patterns
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    # one table, concatenated output
    Y = torch.full((T, D), float("nan"), dtype=dtype, device=DEV)
    tl.tp_embedding(idd, Y, P, E=Ed, bad=bad)
    assert np.array_equal(bits(Y), ref)
    # shard tables in separate allocations (row stride 16 bytes wider than
    # D/P), both outputs
    Ds = D // P
    pad = 8 if dtype == torch.bfloat16 else 4
    shards = []
    for i in range(P):
        buf = torch.zeros((V, Ds + pad), dtype=dtype, device=DEV)
        buf[:, :Ds] = Ed[:, i * Ds:(i + 1) * Ds]
        shards.append(buf[:, :Ds])
    Y2 = torch.full((T, D), float("nan"), dtype=dtype, device=DEV)
    tl.tp_embedding(idd, Y2, P, e_shards=shards, bad=bad)
    assert np.array_equal(bits(Y2), ref)
    Ys = torch.full((P, T, Ds), float("nan"), dtype=dtype, device=DEV)
    tl.tp_embedding(idd, Ys, P, e_shards=shards, y_mode=tl.TP_Y_SHARDS, bad=bad)
    for i in range(P):
        assert np.array_equal(bits(Ys[i]), ref[:, i * Ds:(i + 1) * Ds]), i
    assert int(bad.item()) == 0


def test_embedding_out_of_range_ids():
    V, D, P = 40, 256, 4
    Eb, Ed = _table(7, V, D, torch.bfloat16)
    ids = np.array([0, -1, 39, 40, 5, 1 << 40, 12], dtype=np.int64)
    idd = torch.from_numpy(ids).to(DEV)
    bad = torch.zeros(1, dtype=torch.int32, device=DEV)
    Y = torch.full((ids.size, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_embedding(idd, Y, P, E=Ed, bad=bad)
    assert np.array_equal(bits(Y), oracle.embedding_parallel(ids, Eb, P))
    assert int(bad.item()) == 1


# ---------------------------------------------------------------------------
# Guard cells: the epilogue options write exactly their output view.
# ---------------------------------------------------------------------------

GUARD = [
    # (M, K, N, P, act): narrow and tile paths with whole and ragged tiles, skinny, generic
    (300, 128, 2 * 272, 2, tl.TP_ACT_NONE),
    (300, 128, 2 * 272, 2, tl.TP_ACT_SWIGLU),
    (512, 128, 4 * 256, 4, tl.TP_ACT_SWIGLU),
    (1100, 128, 16 * 512, 16, tl.TP_ACT_SWIGLU),
    (9, 256, 2 * 48, 2, tl.TP_ACT_SWIGLU),
    (9, 256, 2 * 48, 2, tl.TP_ACT_NONE),
    (70, 40, 3 * 12, 3, tl.TP_ACT_SWIGLU),
]


@pytest.mark.parametrize("case", range(len(GUARD)))
@pytest.mark.parametrize("first_col", [8, 1])
def test_epilogue_guard_cells(case, first_col):
    # The output is a view into a wider buffer filled with a sentinel; the view
    # starts at column `first_col` (8: 16-byte aligned rows, vector stores;
    # 1: unaligned, element stores).  Every cell outside the view keeps its
    # bits, and the view equals the call on a dense output.
    M, K, N, P, act = GUARD[case]
    print(f"guard M={M} K={K} N={N} P={P} act={act} first_col={first_col}", flush=True)
    On = N // P // (2 if act == tl.TP_ACT_SWIGLU else 1)
    X = _dev(_ints(990 + case, (M, K)), torch.bfloat16)
    W = _dev(_ints(991 + case, (N, K)), torch.bfloat16)
    b = _dev(_ints(992 + case, (N,), -4, 4), torch.bfloat16)
    sentinel = -12345.0
    buf = torch.full((M + 2, On * P + 16), sentinel, dtype=torch.bfloat16, device=DEV)
    view = buf[1:M + 1, first_col:first_col + On * P]
    tl.tp_linear_column_ex(X, W, view, P, bias=b, act=act)
    dense = torch.empty((M, On * P), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_column_ex(X, W, dense, P, bias=b, act=act)
    torch.cuda.synchronize()
    got = buf.cpu()
    mask = torch.ones_like(got, dtype=torch.bool)
    mask[1:M + 1, first_col:first_col + On * P] = False
    assert torch.all(got[mask] == sentinel), "a cell outside the output view was written"
    assert torch.equal(view.cpu().view(torch.int16), dense.cpu().view(torch.int16))
