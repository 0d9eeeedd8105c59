"""GPU parity on a fixed set of 40 pseudo-random shapes (drawn once from a
seeded generator, the same shapes every run).  Integer-valued inputs keep
every sum exact, so every column and row mode must equal the oracle bit for
bit, as in the parity suite; the shapes mix the decode, tile,
fold-in-registers and generic kernels with ragged M and N and one to four K
steps per shard, in bf16 and fp32."""
import numpy as np
import pytest
import torch

import synth
from gpu_util import bf16_dev, f32_dev
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
