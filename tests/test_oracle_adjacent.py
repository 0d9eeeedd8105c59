"""Pins for the oracle's steps next to the Linear: the column and row bias,
the gated activation of the fused gate+up column layer, the column layer fed
by token slices, and the feature-sharded embedding.  CPU only.

Each check ties the oracle to something other than itself: exact integer
products from numpy, scipy's logistic function, closed forms of silu,
selection weights whose product is known without a matmul, hand-derived
IEEE fold results, and numpy's own row indexing.

A plausible slip fails at least one test here:
  * bias split at the wrong offset, or dropped      -> integer bias tests
  * row bias added per shard, or before the fold    -> fold+bias golden cases, row bias test
  * gate and up halves swapped, or halves of the
    whole weight instead of each shard's            -> selection-weight SwiGLU test
  * silu written as sigmoid, or with a wrong sign   -> silu closed forms and expit
  * embedding shards concatenated out of order      -> tagged-table test
"""
import json
import os

import numpy as np
import pytest
from scipy.special import expit

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _f32(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------------------
# Bias.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,P", [(3, 8, 12, 4), (5, 7, 6, 3), (2, 5, 8, 8), (4, 6, 9, 1)])
def test_column_bias_integer_exact(M, K, N, P):
    X = synth.small_ints(101 + M, (M, K)).astype(np.int64)
    W = synth.small_ints(103 + N, (K, N)).astype(np.int64)
    b = np.arange(N, dtype=np.int64) * 7 - 20        # distinct per output feature
    ref = X @ W + b[None, :]
    got = oracle.column_parallel_linear_bias(X.astype(np.float64), W.astype(np.float64),
                                            b.astype(np.float64), P)
    assert np.array_equal(got, ref.astype(np.float64))


@pytest.mark.parametrize("M,K,N,P", [(3, 8, 12, 4), (5, 9, 6, 3), (2, 16, 4, 8)])
def test_row_bias_integer_exact_and_once(M, K, N, P):
    X = synth.small_ints(107 + M, (M, K)).astype(np.int64)
    W = synth.small_ints(109 + N, (K, N)).astype(np.int64)
    b = np.arange(N, dtype=np.int64) * 3 + 1
    ref = X @ W + b[None, :]                          # the bias counts once, not P times
    got = oracle.row_parallel_linear_bias(X.astype(np.float64), W.astype(np.float64),
                                         b.astype(np.float64), P)
    assert np.array_equal(got, ref.astype(np.float64))


def test_fold_bias_golden_cases():
    cases = json.load(open(os.path.join(GOLDEN, "fold_bias_f32_cases.json")))["cases"]
    assert len(cases) >= 5
    for c in cases:
        parts = np.array([_f32(h) for h in c["parts"]], dtype=np.float32).reshape(-1, 1, 1)
        bias = np.array([_f32(c["bias"])], dtype=np.float32)
        got = oracle.fold_f32(parts, bias)
        assert got.view(np.uint32)[0, 0] == int(c["out"], 16), c["why"]


def test_fold_without_bias_unchanged():
    parts = synth.normal_f32(5, (4, 3, 7))
    a = oracle.fold_f32(parts)
    b = oracle.fold_f32(parts, np.zeros(7, dtype=np.float32))
    # x + 0 == x for every finite x except -0 + 0 = +0: compare values.
    assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# silu and the gated unit.
# ---------------------------------------------------------------------------

def test_silu_closed_forms():
    assert oracle.silu(np.array([0.0]))[0] == 0.0
    # sigmoid(ln 3) = 3 / 4 exactly in real arithmetic.
    assert abs(oracle.silu(np.array([np.log(3.0)]))[0] - 0.75 * np.log(3.0)) < 1e-15
    # silu(x) - silu(-x) = x (sigmoid(x) + sigmoid(-x) = 1).
    x = synth.normal_f32(9, (1000,)).astype(np.float64) * 4
    np.testing.assert_allclose(oracle.silu(x) - oracle.silu(-x), x, rtol=0, atol=1e-14)
    # Limits: silu(40) = 40 in fp64 (sigmoid(40) rounds to 1), silu(-800) = -0.
    assert oracle.silu(np.array([40.0]))[0] == 40.0
    v = oracle.silu(np.array([-800.0]))[0]
    assert v == 0.0 and np.signbit(v)


def test_silu_against_scipy_expit():
    x = synth.normal_f32(10, (4096,)).astype(np.float64) * 6
    np.testing.assert_allclose(oracle.silu(x), x * expit(x), rtol=1e-14, atol=1e-300)


def test_swiglu_gate_then_up():
    # silu(gate) * up: a large gate passes the up value through scaled by the
    # gate; swapping the roles gives a different number.
    assert abs(oracle.swiglu(np.array([30.0]), np.array([1.0]))[0] - 30.0) < 1e-9
    assert abs(oracle.swiglu(np.array([1.0]), np.array([30.0]))[0] - 30.0 * expit(1.0)) < 1e-12
    assert oracle.swiglu(np.array([0.0]), np.array([5.0]))[0] == 0.0


@pytest.mark.parametrize("P", [1, 2, 4])
def test_column_swiglu_selection_weights(P):
    # Selection weights: gate feature h reads X column a[h], up feature h reads
    # X column c[h], so G = X[:, a] + b_gate and U = X[:, c] + b_up exactly,
    # and H = silu(G) * U is known without any matmul.  The fused weight is
    # laid out shard by shard, [gate_i | up_i] per shard.
    rng = np.random.default_rng(31 + P)
    M, K, I = 6, 10, 8
    X = synth.small_ints(41, (M, K)).astype(np.float64) + 0.25
    a = rng.integers(0, K, size=I)
    c = rng.integers(0, K, size=I)
    bg = np.linspace(-1, 1, I)
    bu = np.linspace(2, -2, I)
    s = I // P
    W = np.zeros((K, 2 * I))
    b = np.zeros(2 * I)
    for i in range(P):
        base = 2 * s * i
        for h in range(s):
            hh = i * s + h
            W[a[hh], base + h] = 1.0
            W[c[hh], base + s + h] = 1.0
            b[base + h] = bg[hh]
            b[base + s + h] = bu[hh]
    G = X[:, a] + bg[None, :]
    U = X[:, c] + bu[None, :]
    exp = G * expit(G) * U
    g, u = oracle.column_parallel_gate_up(X, W, b, P)
    assert np.array_equal(g, G) and np.array_equal(u, U)
    np.testing.assert_allclose(oracle.column_parallel_swiglu(X, W, b, P), exp,
                               rtol=1e-14, atol=1e-14)


# ---------------------------------------------------------------------------
# Column layer on all-gathered token slices.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("M,K,N,P", [(8, 6, 12, 4), (6, 5, 6, 3), (16, 8, 8, 8)])
def test_gathered_column_integer_exact(M, K, N, P):
    X = synth.small_ints(201 + M, (M, K)).astype(np.int64)
    W = synth.small_ints(203 + N, (K, N)).astype(np.int64)
    slices = [X[j * (M // P):(j + 1) * (M // P)].astype(np.float64) for j in range(P)]
    got = oracle.column_parallel_linear_gathered(slices, W.astype(np.float64), P)
    assert np.array_equal(got, (X @ W).astype(np.float64))


# ---------------------------------------------------------------------------
# Embedding sharded on its feature dim.
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("P", [1, 2, 4, 8])
def test_embedding_tagged_table(P):
    # E[v, d] = v * D + d: every output value names the row and feature it
    # came from, so a wrong row, a wrong shard order or a wrong offset shows.
    V, D, T = 37, 16, 50
    E = (np.arange(V)[:, None] * D + np.arange(D)[None, :]).astype(np.float32)
    ids = np.random.default_rng(P).integers(0, V, size=T)
    got = oracle.embedding_parallel(ids, E, P)
    assert got.dtype == np.float32
    exp = (ids[:, None] * D + np.arange(D)[None, :]).astype(np.float32)
    assert np.array_equal(got, exp)
    assert np.array_equal(got, E[ids])                 # numpy's own row indexing


def test_embedding_out_of_range_ids_give_zero_rows():
    V, D = 5, 8
    E = np.arange(V * D, dtype=np.float32).reshape(V, D) + 1
    ids = np.array([0, -1, 4, 5, 2, 1 << 40])
    got = oracle.embedding_parallel(ids, E, 4)
    for t, v in enumerate(ids):
        if 0 <= v < V:
            assert np.array_equal(got[t], E[v])
        else:
            assert np.all(got[t] == 0)


def test_embedding_bf16_bits_copied():
    # A lookup copies bit patterns: bf16 patterns (uint16) come through as is.
    E = synth.normal_bf16(3, (11, 24), 1.0)
    ids = np.array([3, 0, 10, 3])
    got = oracle.embedding_parallel(ids, E, 3)
    assert got.dtype == np.uint16
    assert np.array_equal(got, E[ids])
