"""GPU parity on a fixed set of 40 pseudo-random shapes (drawn once from a
seeded generator, the same shapes every run).  Integer-valued inputs keep
every sum exact, so every column and row mode must equal the oracle bit for
bit, as in the parity suite; the shapes mix the decode, tile,
fold-in-registers and generic kernels with ragged M and N and one to four K
steps per shard, in bf16 and fp32.  On N(0,1) x N(0, 0.02^2) data, where
rounding happens in every sum, the fused fold and the one-call
reduce-scatter must still equal partials + fold bit for bit (the same fp32
operations in the same order), both where the library picks the way to fold
and with every shape a fused kernel takes sent to it."""
import numpy as np
import pytest
import torch

import synth
import tensor_linear_amd as tl
from gpu_util import DEV, FOLD_POLICIES, bf16_dev, bits, f32_dev, row_fold, workspace
from test_gpu_parity import _run_all_modes

pytestmark = pytest.mark.gpu


def _shapes(n=40, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(n):
        P = int(rng.choice([1, 2, 3, 4, 8]))
        M = int(rng.choice([rng.integers(1, 65), rng.integers(65, 301), rng.choice([256, 512])]))
        ks = int(rng.choice([1, 3, 8, 64, 72, 128, 192, 256]))
        ns = int(rng.choice([rng.integers(1, 41), rng.integers(100, 301), rng.choice([128, 256])]))
        dt = "f32" if rng.random() < 0.25 else "bf16"
        out.append((M, ks * P, ns * P, P, dt, int(rng.integers(0, 10**6))))
    return out


SHAPES = _shapes()


@pytest.mark.parametrize("case", range(len(SHAPES)))
def test_random_shapes_bitwise(case):
    M, K, N, P, dt, seed = SHAPES[case]
    print(f"case M={M} K={K} N={N} P={P} {dt} seed={seed}", flush=True)
    X = synth.small_ints(seed, (M, K))
    W = synth.small_ints(seed + 1, (N, K))
    if dt == "bf16":
        Xd, Wd, dtype = bf16_dev(synth.to_bf16_bits(X)), bf16_dev(synth.to_bf16_bits(W)), torch.bfloat16
    else:
        Xd, Wd, dtype = f32_dev(X), f32_dev(W), torch.float32
    _run_all_modes(Xd, Wd, X.astype(np.float64), W.T.astype(np.float64), M, K, N, P, dtype)


@pytest.mark.parametrize("case", [i for i, s in enumerate(SHAPES) if s[4] == "bf16"])
def test_random_shapes_fused_equals_sum(case):
    M, K, N, P, dt, seed = SHAPES[case]
    print(f"case M={M} K={K} N={N} P={P} seed={seed}", flush=True)
    X = bf16_dev(synth.to_bf16_bits(synth.normal_f32(seed, (M, K))))
    W = bf16_dev(synth.to_bf16_bits(synth.normal_f32(seed + 1, (N, K), 0.02)))
    Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row(X, W, Y, P, tl.TP_ROW_SUM, workspace(tl.TP_ROW_SUM, M, N, P))
    ref = bits(Y)
    modes = [tl.TP_ROW_FUSED] + ([tl.TP_ROW_SCATTER] if M % P == 0 else [])
    for policy in FOLD_POLICIES:
        with row_fold(policy):
            for mode in modes:
                Y = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
                tl.tp_linear_row(X, W, Y, P, mode, workspace(mode, M, N, P))
                assert np.array_equal(bits(Y), ref), f"mode {mode} {policy}"
