"""Property tests of the oracle on random small shapes (hypothesis).

Integer-valued operands keep every product and sum exact in fp64, so the
tensor-parallel forms must equal numpy's exact int64 product bit for bit:
the column concatenation, each column shard, the row sum and each row
partial, and the reduce-scatter followed by the all-gather ("模型并行",
"Tensor-parallel 线性层"; the Shard(0) slices of "DTensor API 文档", "放置策略类型").  The fp32
fold is one IEEE add at a time in ascending shard order, which numpy's own
float32 adds reproduce exactly, special values included.
"""
import numpy as np
from hypothesis import given, settings, strategies as st

import oracle


@st.composite
def tp_problem(draw):
    P = draw(st.integers(1, 4))
    M = draw(st.integers(1, 9))
    K = P * draw(st.integers(1, 5))
    N = P * draw(st.integers(1, 5))
    seed = draw(st.integers(0, 2**31 - 1))
    rng = np.random.default_rng(seed)
    X = rng.integers(-3, 4, size=(M, K))
    W_io = rng.integers(-3, 4, size=(K, N))
    return P, X, W_io


@settings(max_examples=150, deadline=None)
@given(tp_problem())
def test_parallel_forms_equal_exact_product(prob):
    P, X, W_io = prob
    exact = (X.astype(np.int64) @ W_io.astype(np.int64)).astype(np.float64)
    Xf, Wf = X.astype(np.float64), W_io.astype(np.float64)
    assert np.array_equal(oracle.dense(Xf, Wf), exact)
    assert np.array_equal(oracle.column_parallel_linear(Xf, Wf, P), exact)
    n = W_io.shape[1] // P
    for i, yi in enumerate(oracle.column_shards(Xf, Wf, P)):
        assert np.array_equal(yi, exact[:, i * n:(i + 1) * n])
    k = X.shape[1] // P
    parts = oracle.row_partials(Xf, Wf, P)
    assert len(parts) == P
    for i, p in enumerate(parts):
        ref = X[:, i * k:(i + 1) * k].astype(np.int64) @ W_io[i * k:(i + 1) * k].astype(np.int64)
        assert np.array_equal(p, ref.astype(np.float64))
    assert np.array_equal(oracle.row_parallel_linear(Xf, Wf, P), exact)


@settings(max_examples=100, deadline=None)
@given(tp_problem())
def test_reduce_scatter_then_all_gather(prob):
    P, X, W_io = prob
    M = X.shape[0]
    if M % P:
        X = np.concatenate([X] * P, axis=0)      # make the token count divisible
    Xf, Wf = X.astype(np.float64), W_io.astype(np.float64)
    parts = oracle.row_partials(Xf, Wf, P)
    slices = oracle.reduce_scatter_rows(parts, P)
    s = X.shape[0] // P
    exact = (X.astype(np.int64) @ W_io.astype(np.int64)).astype(np.float64)
    assert len(slices) == P
    for j, sl in enumerate(slices):
        assert np.array_equal(sl, exact[j * s:(j + 1) * s])
    assert np.array_equal(oracle.all_gather_rows(slices), exact)


_f32 = st.floats(width=32, allow_nan=True, allow_infinity=True, allow_subnormal=True)


@settings(max_examples=200, deadline=None)
@given(st.integers(1, 6), st.integers(1, 4), st.integers(1, 5), st.data())
def test_fold_f32_is_sequential_ieee_adds(P, M, N, data):
    vals = data.draw(st.lists(_f32, min_size=P * M * N, max_size=P * M * N))
    parts = np.array(vals, dtype=np.float32).reshape(P, M, N)
    acc = parts[0].copy()
    with np.errstate(all="ignore"):
        for i in range(1, P):
            acc = (acc + parts[i]).astype(np.float32)
    got = oracle.fold_f32(parts)
    both_nan = np.isnan(got) & np.isnan(acc)
    assert np.array_equal(got.view(np.uint32)[~both_nan], acc.view(np.uint32)[~both_nan])
    assert np.array_equal(np.isnan(got), np.isnan(acc))
