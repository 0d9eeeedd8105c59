"""Many shards (P = 16, 32, 64 = TP_MAX_SHARDS) through every entry point, bit for
bit against the oracle on integer-valued inputs (every sum exact in fp32):
column (tile and skinny kernels, both output layouts), row in every mode
(tile partials + fold, the fused decode and prefill folds, the
reduce-scatter), the column layer on P slice allocations, and the
embedding with P shard tables."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import DEV, bf16_dev, bits, expected_bits, workspace

pytestmark = pytest.mark.gpu


def _ints(seed, shape):
    return synth.small_ints(seed, shape)


def _dev(a):
    return bf16_dev(synth.to_bf16_bits(np.asarray(a, dtype=np.float32)))


@pytest.mark.parametrize("P", [16, 32, 64])
@pytest.mark.parametrize("M", [16, 512])
def test_many_shards_bitwise(P, M):
    K, N = 64 * P, 16 * P            # K/P = 64 (one tile K step), N/P = 16
    print(f"many shards P={P} M={M} K={K} N={N}", flush=True)
    X, W = _ints(300 + P, (M, K)), _ints(301 + P, (N, K))
    Xd, Wd = _dev(X), _dev(W)
    X64, Wio = X.astype(np.float64), W.T.astype(np.float64)
    dt = torch.bfloat16
    # column, concatenated and as shard blocks
    Y = torch.full((M, N), float("nan"), dtype=dt, device=DEV)
    tl.tp_linear_column(Xd, Wd, Y, P)
    ref = oracle.column_parallel_linear(X64, Wio, P)
    assert np.array_equal(bits(Y), expected_bits(ref, dt)), "column"
    Ys = torch.full((P, M, N // P), float("nan"), dtype=dt, device=DEV)
    tl.tp_linear_column(Xd, Wd, Ys, P, tl.TP_Y_SHARDS)
    for i in range(P):
        assert np.array_equal(bits(Ys[i]), expected_bits(ref[:, i * 16:(i + 1) * 16], dt)), i
    # row, every mode
    ref = oracle.row_parallel_linear(X64, Wio, P)
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED, tl.TP_ROW_SCATTER):
        if mode == tl.TP_ROW_SCATTER and M % P:
            continue
        Y = torch.full((M, N), float("nan"), dtype=dt, device=DEV)
        tl.tp_linear_row(Xd, Wd, Y, P, mode, workspace(mode, M, N, P))
        assert np.array_equal(bits(Y), expected_bits(ref, dt)), f"row mode {mode}"
    # the column layer on P slice allocations
    s = M // P
    if M % P == 0:
        slices = [Xd[j * s:(j + 1) * s].clone() for j in range(P)]
        Y = torch.full((M, N), float("nan"), dtype=dt, device=DEV)
        tl.tp_linear_column_ex(None, Wd, Y, P, x_slices=slices)
        ref = oracle.column_parallel_linear_gathered([X64[j * s:(j + 1) * s] for j in range(P)], Wio, P)
        assert np.array_equal(bits(Y), expected_bits(ref, dt)), "gathered column"


@pytest.mark.parametrize("P", [16, 64])
def test_many_shard_embedding(P):
    V, D, T = 300, 8 * P, 77
    E = synth.normal_bf16(400 + P, (V, D))
    ids = np.random.default_rng(P).integers(0, V, size=T)
    Ds = D // P
    shards = [bf16_dev(np.ascontiguousarray(E[:, i * Ds:(i + 1) * Ds])) for i in range(P)]
    Y = torch.full((T, D), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_embedding(torch.from_numpy(ids.astype(np.int64)).to(DEV), Y, P, e_shards=shards)
    assert np.array_equal(bits(Y), oracle.embedding_parallel(ids, E, P))
