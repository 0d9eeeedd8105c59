"""GPU parity with row strides whose byte offsets pass 2^32.

X or W is a column view of a buffer whose rows are so far apart that the
view spans more than 4 GiB.  The tile kernels address a tile's rows with
32-bit offsets and must not take such views: the launch falls back to the
generic kernel (M > 48) or takes the decode kernel, whose addresses are
64-bit (M <= 48).  Every column and row mode is checked bit for bit against
the oracle on integer inputs (all sums exact in fp32), as in the parity suite.
"""
import numpy as np
import pytest
import torch

import synth
from gpu_util import DEV, bf16_dev
from test_gpu_parity import _run_all_modes

pytestmark = pytest.mark.gpu

# (M, K, N, P, which operand is the strided view)
CASES = [
    (264, 128, 256, 2, "x"),   # tile-sized M: generic kernel; ragged M tile
    (16, 128, 96, 2, "x"),     # decode kernel, 64-bit row addresses
    (264, 128, 256, 2, "w"),   # W rows far apart: generic kernel
    (16, 256, 256, 4, "w"),    # decode kernel
]


def _row_stride(rows: int) -> int:
    """Elements per row of the backing buffer: the last row starts just past
    byte 2^32 of it."""
    return ((1 << 32) // (2 * (rows - 1)) // 64 + 1) * 64


def _strided(bits2d: np.ndarray) -> torch.Tensor:
    rows, cols = bits2d.shape
    full = torch.zeros((rows, _row_stride(rows)), dtype=torch.bfloat16, device=DEV)
    full[:, :cols] = bf16_dev(bits2d)
    return full[:, :cols]


@pytest.mark.parametrize("case", range(len(CASES)))
def test_large_row_strides_bitwise(case):
    M, K, N, P, which = CASES[case]
    ld = _row_stride(M if which == "x" else N)
    print(f"case M={M} K={K} N={N} P={P} strided {which}, row stride {ld}", flush=True)
    X = synth.small_ints(900 + 2 * case, (M, K))
    W = synth.small_ints(901 + 2 * case, (N, K))
    xb, wb = synth.to_bf16_bits(X), synth.to_bf16_bits(W)
    Xd = _strided(xb) if which == "x" else bf16_dev(xb)
    Wd = _strided(wb) if which == "w" else bf16_dev(wb)
    view = Xd if which == "x" else Wd
    assert view.stride(0) == ld and (view.shape[0] - 1) * ld * 2 > (1 << 32)
    _run_all_modes(Xd, Wd, X.astype(np.float64), W.T.astype(np.float64), M, K, N, P,
                   torch.bfloat16)
    del Xd, Wd, view
    torch.cuda.empty_cache()
