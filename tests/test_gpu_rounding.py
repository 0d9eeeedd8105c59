"""The device's one rounding, fp32 -> bf16, against the oracle's
round-to-nearest-even ("bfloat16" format: 8 exponent bits, 7 stored mantissa
bits; the fold's result is rounded once to the output type).

  * every one of the 2^32 fp32 bit patterns, through the shard fold with
    P = 1 (the fold of one part is that part, then the rounding), compared
    with the oracle's RNE; a NaN input must give a NaN (its payload is not
    fixed), and the fp32 output of a one-part fold is the input itself;
  * the GEMM epilogues: values v with any 24-bit mantissa are built as
    v = a + b + c from three bf16 pieces (the top, middle and low 8
    significant bits), so the fp32 accumulator holds v exactly whatever the
    summation order; the kernels must then round v exactly as the oracle
    does, ties, overflow to infinity and both signs included.
"""
import numpy as np
import pytest
import torch

import oracle
import tensor_linear_amd as tl
from gpu_util import DEV, bf16_dev, bits, expected_bits, workspace

pytestmark = pytest.mark.gpu

CHUNK_LOG2 = 26


def _is_nan32(u):
    return (u & np.uint32(0x7FFFFFFF)) > np.uint32(0x7F800000)


def _is_nan16(h):
    return (h & np.uint16(0x7FFF)) > np.uint16(0x7F80)


def test_fold_rounds_every_fp32_pattern():
    n = 1 << CHUNK_LOG2
    side = 1 << (CHUNK_LOG2 // 2)
    Y = torch.empty((side, side), dtype=torch.bfloat16, device=DEV)
    Yf = torch.empty((side, side), dtype=torch.float32, device=DEV)
    ramp_dev = torch.arange(n, dtype=torch.int32, device=DEV)
    ramp_host = np.arange(n, dtype=np.uint32)
    bad = 0
    for c in range(1 << (32 - CHUNK_LOG2)):
        start = c * n
        s32 = start if start < (1 << 31) else start - (1 << 32)
        part = (ramp_dev + s32).view(torch.float32).view(1, side, side)
        tl.tp_shard_reduce(part, Y, 1)
        u = ramp_host + np.uint32(start)
        want = oracle.round_bf16(u.view(np.float32))
        got = bits(Y).ravel()
        nan = _is_nan32(u)
        ok = np.where(nan, _is_nan16(got), got == want)
        if not ok.all():
            idx = np.flatnonzero(~ok)[:8]
            print(f"chunk {c}: {np.count_nonzero(~ok)} mismatches, e.g. " +
                  ", ".join(f"{u[i]:#010x}->{got[i]:#06x} (want {want[i]:#06x})" for i in idx),
                  flush=True)
            bad += np.count_nonzero(~ok)
        if c % 16 == 0 or c in (31, 32, 63):
            # fp32 output of a one-part fold: the input bits (NaNs aside)
            tl.tp_shard_reduce(part, Yf, 1)
            gf = bits(Yf).ravel()
            assert np.all(np.where(nan, _is_nan32(gf), gf == u)), f"fp32 identity, chunk {c}"
    assert bad == 0, f"{bad} fp32 patterns rounded differently from RNE"


def _values(rng, n):
    """fp32 values whose three bf16 pieces are normal or zero: exponent field
    in [27, 254], random sign and mantissa, with the low 16 bits forced to
    the rounding boundaries (ties with even and odd kept bit, one below and
    one above a tie, exact) for half of them, and the largest finite values
    (which round to infinity or to the largest bf16)."""
    e = rng.integers(27, 255, size=n, dtype=np.uint32)
    man = rng.integers(0, 1 << 23, size=n, dtype=np.uint32)
    sgn = rng.integers(0, 2, size=n, dtype=np.uint32)
    u = (sgn << 31) | (e << 23) | man
    special = np.array([0x0000, 0x7FFF, 0x8000, 0x8001, 0xFFFF, 0x0001], dtype=np.uint32)
    pick = rng.integers(0, 2, size=n).astype(bool)
    u = np.where(pick, (u & np.uint32(0xFFFF0000)) | special[rng.integers(0, 6, size=n)], u)
    edge = np.array([0x7F7F7FFF, 0x7F7F8000, 0x7F7F8001, 0x7F7FFFFF, 0x7F7EFFFF, 0x7F7E8000,
                     0x7F7E8001, 0x0D808000, 0x0D818000, 0x3F808000, 0x3F818000],
                    dtype=np.uint32)
    edge = np.concatenate([edge, edge | np.uint32(0x80000000)])
    u[: edge.size] = edge
    return u.view(np.float32)


def _pieces(v):
    """v = a + b + c with a, b, c bf16: a keeps v's top 16 bits, b the top
    16 bits of the remainder, c the rest (at most 8 significant bits)."""
    mask = np.uint32(0xFFFF0000)
    a = (v.view(np.uint32) & mask).view(np.float32)
    r = v - a
    b = (r.view(np.uint32) & mask).view(np.float32)
    c = r - b
    for p in (a, b, c):
        assert np.all((p.view(np.uint32) & np.uint32(0xFFFF)) == 0)
    assert np.array_equal(a.astype(np.float64) + b + c, v.astype(np.float64))
    return a, b, c


def _gemm_inputs(M, KS, N, seed):
    """X [M, 3 KS] picks, in row m, column t = m % T of each of the three
    K regions (T = min(KS, M)); W [N, 3 KS] holds piece j of value v[n, t] in
    region j.  So (X W^T)[m, n] = v[n, m % T] exactly."""
    T = min(KS, M)
    rng = np.random.default_rng(seed)
    v = _values(rng, N * T).reshape(N, T)
    pieces = _pieces(v.ravel())
    W = np.zeros((N, 3 * KS), dtype=np.float32)
    for j, p in enumerate(pieces):
        W[:, j * KS: j * KS + T] = p.reshape(N, T)
    X = np.zeros((M, 3 * KS), dtype=np.float32)
    for m in range(M):
        X[m, [m % T, KS + m % T, 2 * KS + m % T]] = 1.0
    to_bits = lambda a: (a.view(np.uint32) >> 16).astype(np.uint16)   # exact: low halves are 0
    return (bf16_dev(to_bits(X)), bf16_dev(to_bits(W)),
            X.astype(np.float64), W.T.astype(np.float64))


# (label, M, KS, N): M > 48 and KS % 64 == 0 reach the tile kernels, M <= 48
# the skinny kernel (and the fused fold), KS = 72 the generic kernel.
GEMM_CASES = [("tile", 128, 64, 4096), ("skinny-m48", 48, 64, 4096), ("narrow-m64", 64, 64, 4096),
              ("skinny-m16", 16, 64, 8192), ("generic", 128, 72, 2048)]


@pytest.mark.parametrize("case", GEMM_CASES, ids=[c[0] for c in GEMM_CASES])
def test_gemm_epilogue_rounding(case):
    label, M, KS, N = case
    print(f"{label}: M={M} K={3 * KS} N={N}", flush=True)
    X, W, X64, Wio = _gemm_inputs(M, KS, N, seed=len(label) * 31 + M)
    for P in (1, 4):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_column(X, W, Y, P)
        want = expected_bits(oracle.column_parallel_linear(X64, Wio, P), torch.bfloat16)
        got = bits(Y)
        assert np.array_equal(got, want), \
            f"column P={P}: {np.count_nonzero(got != want)} of {got.size} differ"
    # Row-parallel with P = 3: part j is piece j, the fold adds them.
    want = expected_bits(oracle.row_parallel_linear(X64, Wio, 3), torch.bfloat16)
    for mode in (tl.TP_ROW_SUM, tl.TP_ROW_FUSED):
        Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
        tl.tp_linear_row(X, W, Y, 3, mode, workspace(mode, M, N, 3))
        got = bits(Y)
        assert np.array_equal(got, want), \
            f"row mode {mode}: {np.count_nonzero(got != want)} of {got.size} differ"
