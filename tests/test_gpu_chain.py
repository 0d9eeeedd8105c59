"""The Megatron pairing of the two forms ("Module 并行：实现 DP/TP/CP/PP 组合",
"Tensor Parallel": fc1 column-parallel, Replicate in, Shard on the feature
dim out; fc2 row-parallel, Shard in, all-reduced to Replicate out): the
column layer's output, whose P column blocks are exactly the row layer's P
input shards, goes straight into the row layer with no exchange.  Compared
with the oracle's own chain (its bf16-rounded fc1 output into its fc2) and
with the dense (X W1) W2, on every row mode."""
import numpy as np
import pytest
import torch

import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import DEV, bf16_dev, to_f64, workspace

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("M,H,I,P", [(264, 1024, 4096, 8), (16, 2048, 4096, 8), (300, 512, 1536, 3)])
def test_column_then_row_chain(M, H, I, P):
    print(f"chain M={M} H={H} I={I} P={P}", flush=True)
    X = synth.normal_bf16(600 + M, (M, H), synth.SIGMA_X)
    W1 = synth.normal_bf16(601 + M, (I, H), synth.SIGMA_W)
    W2 = synth.normal_bf16(602 + M, (H, I), synth.SIGMA_W)
    Xd, W1d, W2d = bf16_dev(X), bf16_dev(W1), bf16_dev(W2)
    Y1 = torch.empty((M, I), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_column(Xd, W1d, Y1, P)
    X64, W1io, W2io = oracle.widen_bf16(X), oracle.widen_bf16(W1).T, oracle.widen_bf16(W2).T
    y1 = oracle.column_parallel_linear(X64, W1io, P)
    y1_bf16 = oracle.widen_bf16(oracle.round_bf16(y1.astype(np.float32)))
    ref = oracle.row_parallel_linear(y1_bf16, W2io, P)
    dense = oracle.dense(oracle.dense(X64, W1io), W2io)
    sy = float(np.sqrt(np.mean(y1_bf16 ** 2)))
    tol = 2e-2 * np.sqrt(I) * sy * synth.SIGMA_W
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED, tl.TP_ROW_SCATTER):
        if mode == tl.TP_ROW_SCATTER and M % P:
            continue
        Y2 = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_row(Y1, W2d, Y2, P, mode, workspace(mode, M, H, P))
        got = to_f64(Y2)
        # The dense reference skips the rounding of fc1's output to bf16, a
        # second error of the same size as the bar: twice the bar there.
        for name, r, bar in (("oracle chain", ref, tol), ("dense (X W1) W2", dense, 2 * tol)):
            e, m = oracle.rel_l2(got, r), oracle.max_abs(got, r)
            print(f"  mode {mode} vs {name}: rel_l2={e:.3e} max_abs={m:.3e} (bar {bar:.3e})", flush=True)
            assert e <= 1e-2 and m <= bar, (mode, name)
