"""Pins for the CPU oracle: each check ties it to something other than
itself (a value printed on the pages, a closed form, an invariant, a library
routine written by someone else, or hand-derived IEEE results).  CPU only.

A plausible slip in the oracle fails at least one test here:
  * a dropped or repeated shard in the row sum   -> integer exactness, identity W
  * a transposed operand                         -> one-hot W, non-square integer checks
  * a wrong split offset or chunk size           -> index-map tests, identity W
  * a wrong fold order or extra rounding         -> the fold golden cases
  * a wrong rounding rule                        -> the bf16 golden cases
  * a slip in the comparison metrics (a dropped square root, the norm of
    the result instead of the reference's, a signed maximum, swapped
    arguments, silent broadcasting)              -> the metric closed forms
"""
import json
import os

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _hex_f32(h):
    return np.array([int(h, 16)], dtype=np.uint32).view(np.float32)[0]


# ---------------------------------------------------------------------------
# Worked example ("模型并行", section "Tensor-parallel 线性层"): seed 0, x then
# weight drawn with torch.randn on the CPU, P = 4; both parallel forms must
# match the dense product and the column result has shape (3, 12).
# ---------------------------------------------------------------------------

def _worked_example():
    import torch
    torch.manual_seed(0)
    x, weight = torch.randn(3, 8), torch.randn(8, 12)
    return x, weight


def test_worked_example_page_checks():
    import torch
    x, w = _worked_example()
    dense_t = x @ w                              # torch's own matmul, fp32
    X = oracle.widen_f32(x.numpy())
    W = oracle.widen_f32(w.numpy())
    col = oracle.column_parallel_linear(X, W, 4)
    row = oracle.row_parallel_linear(X, W, 4)
    assert col.shape == (3, 12)
    torch.testing.assert_close(torch.from_numpy(col.astype(np.float32)), dense_t)
    torch.testing.assert_close(torch.from_numpy(row.astype(np.float32)), dense_t)


def test_worked_example_fp64_against_numpy():
    x, w = _worked_example()
    X = oracle.widen_f32(x.numpy())
    W = oracle.widen_f32(w.numpy())
    ref = X @ W                                   # numpy fp64 matmul
    for got in (oracle.dense(X, W), oracle.column_parallel_linear(X, W, 4),
                oracle.row_parallel_linear(X, W, 4)):
        np.testing.assert_allclose(got, ref, rtol=1e-13, atol=1e-13)


# ---------------------------------------------------------------------------
# Brute force on small integer-valued inputs: every sum is exact, so the
# oracle must agree bit for bit with numpy's int64 matmul.
# ---------------------------------------------------------------------------

SHAPES = [(1, 1, 1, 1), (2, 4, 6, 2), (3, 8, 12, 4), (5, 6, 9, 3), (4, 16, 8, 8),
          (7, 10, 5, 5), (3, 12, 12, 1), (2, 15, 9, 3)]


@pytest.mark.parametrize("M,K,N,P", SHAPES)
def test_integer_inputs_exact(M, K, N, P):
    X = synth.small_ints(11 + M, (M, K)).astype(np.int64)
    W = synth.small_ints(23 + N, (K, N)).astype(np.int64)
    ref = X @ W                                   # exact integer product
    got_dense = oracle.dense(X.astype(np.float64), W.astype(np.float64))
    assert np.array_equal(got_dense, ref.astype(np.float64))
    if N % P == 0:
        got = oracle.column_parallel_linear(X.astype(np.float64), W.astype(np.float64), P)
        assert np.array_equal(got, ref.astype(np.float64))
        shards = oracle.column_shards(X.astype(np.float64), W.astype(np.float64), P)
        s = N // P
        for i, yi in enumerate(shards):
            assert np.array_equal(yi, (X @ W[:, i * s:(i + 1) * s]).astype(np.float64))
    if K % P == 0:
        got = oracle.row_parallel_linear(X.astype(np.float64), W.astype(np.float64), P)
        assert np.array_equal(got, ref.astype(np.float64))
        parts = oracle.row_partials(X.astype(np.float64), W.astype(np.float64), P)
        s = K // P
        assert len(parts) == P
        for i, yp in enumerate(parts):
            assert np.array_equal(yp, (X[:, i * s:(i + 1) * s] @ W[i * s:(i + 1) * s]).astype(np.float64))


def test_column_concat_equals_dense_bitwise():
    # Each column of the concatenation is the same k-ascending fp64 sum as
    # the dense product: equal bit for bit, not just within a tolerance.
    X = oracle.widen_f32(synth.normal_f32(1, (9, 40)))
    W = oracle.widen_f32(synth.normal_f32(2, (40, 24), 0.02))
    assert np.array_equal(oracle.column_parallel_linear(X, W, 8), oracle.dense(X, W))


def test_row_sum_within_reassociation_bound():
    # Row parallel reorders the fp64 sum; it must stay within the classic
    # bound |err| <= gamma_K * sum_k |x_k||w_k|, gamma_K = K u / (1 - K u).
    K = 64
    X = oracle.widen_f32(synth.normal_f32(3, (7, K)))
    W = oracle.widen_f32(synth.normal_f32(4, (K, 16), 0.02))
    u = 2.0 ** -53
    gamma = K * u / (1 - K * u)
    bound = 2 * gamma * (np.abs(X) @ np.abs(W))
    for P in (1, 2, 4, 8, 16):
        diff = np.abs(oracle.row_parallel_linear(X, W, P) - X @ W)
        assert np.all(diff <= bound)


def test_identity_weight():
    # W = I: column shard i is X's column block i; the row sum returns X.
    X = synth.small_ints(5, (6, 12)).astype(np.float64) + 0.5
    I = np.eye(12)
    for P in (1, 2, 3, 4, 6, 12):
        shards = oracle.column_shards(X, I, P)
        s = 12 // P
        for i, yi in enumerate(shards):
            assert np.array_equal(yi, X[:, i * s:(i + 1) * s])
        assert np.array_equal(oracle.row_parallel_linear(X, I, P), X)
        parts = oracle.row_partials(X, I, P)
        for i, yp in enumerate(parts):
            exp = np.zeros_like(X)
            exp[:, i * s:(i + 1) * s] = X[:, i * s:(i + 1) * s]
            assert np.array_equal(yp, exp)


def test_one_hot_weight_selects_columns():
    # W[:, n] = e_{perm[n]} (K != N): Y[:, n] = X[:, perm[n]].  A transposed
    # operand or a swapped index cannot pass this.
    rng = np.random.default_rng(7)
    M, K, N = 5, 6, 10
    X = rng.standard_normal((M, K))
    perm = rng.integers(0, K, size=N)
    W = np.zeros((K, N))
    W[perm, np.arange(N)] = 1.0
    exp = X[:, perm]
    assert np.array_equal(oracle.dense(X, W), exp)
    assert np.array_equal(oracle.column_parallel_linear(X, W, 5), exp)
    assert np.array_equal(oracle.row_parallel_linear(X, W, 3), exp)


def test_rank_one_closed_form():
    # X = a b^T, W = c d^T  ->  Y = a (b . c) d^T, exact for integers.
    a = np.array([1., -2., 3.])
    b = np.array([2., 0., -1., 1., 2., -2.])
    c = np.array([1., 1., -2., 0., 3., 1.])
    d = np.array([1., -1., 2., 0.])
    X, W = np.outer(a, b), np.outer(c, d)
    exp = np.outer(a, d) * float(b @ c)
    for P in (1, 2, 3, 6):
        assert np.array_equal(oracle.row_parallel_linear(X, W, P), exp)
    for P in (1, 2, 4):
        assert np.array_equal(oracle.column_parallel_linear(X, W, P), exp)


def test_transpose_relation():
    X = synth.small_ints(8, (4, 7)).astype(np.float64)
    W = synth.small_ints(9, (7, 5)).astype(np.float64)
    assert np.array_equal(oracle.dense(W.T, X.T), oracle.dense(X, W).T)


def test_indivisible_split_rejected():
    # The page's reference asserts divisibility before splitting.
    X = np.zeros((3, 8))
    W = np.zeros((8, 12))
    with pytest.raises(ValueError):
        oracle.column_parallel_linear(X, W, 5)
    with pytest.raises(ValueError):
        oracle.row_parallel_linear(X, W, 3)
    with pytest.raises(ValueError):
        oracle.split(X, 0, 0)


def test_reduce_scatter_then_all_gather():
    X = synth.small_ints(12, (8, 6)).astype(np.float64)
    W = synth.small_ints(13, (6, 4)).astype(np.float64)
    parts = oracle.row_partials(X, W, 2)
    slices = oracle.reduce_scatter_rows(parts, 4)
    ref = X @ W
    assert len(slices) == 4
    for j, s in enumerate(slices):
        assert np.array_equal(s, ref[2 * j:2 * j + 2])
    assert np.array_equal(oracle.all_gather_rows(slices), ref)


# ---------------------------------------------------------------------------
# fp32 fold: hand-derived IEEE cases (order and rounding matter) and numpy's
# own float32 adds on random data.
# ---------------------------------------------------------------------------

def test_fold_f32_golden_cases():
    with open(os.path.join(GOLDEN, "fold_f32_cases.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        parts = np.array([_hex_f32(h) for h in c["parts"]], dtype=np.float32)
        got = oracle.fold_f32(parts.reshape(len(parts), 1, 1))[0, 0]
        want = np.uint32(int(c["fold"], 16))
        assert got.view(np.uint32) == want, c["why"]


def test_fold_f32_matches_numpy_sequential_adds():
    P, M, N = 8, 37, 53
    parts = synth.normal_f32(99, (P, M, N)) * np.float32(1e3)
    acc = parts[0].copy()
    for i in range(1, P):
        acc = np.add(acc, parts[i], dtype=np.float32)
    got = oracle.fold_f32(parts)
    assert np.array_equal(got.view(np.uint32), acc.view(np.uint32))


# ---------------------------------------------------------------------------
# bf16 rounding: hand-derived bit cases and torch's CPU cast.
# ---------------------------------------------------------------------------

def test_bf16_golden_cases():
    with open(os.path.join(GOLDEN, "bf16_rne_cases.json")) as f:
        g = json.load(f)
    src = np.array([int(c["f32"], 16) for c in g["cases"]], dtype=np.uint32)
    want = np.array([int(c["bf16"], 16) for c in g["cases"]], dtype=np.uint16)
    got = oracle.round_bf16(src.view(np.float32))
    for s, w, o, c in zip(src, want, got, g["cases"]):
        assert o == w, f"{hex(s)} -> {hex(o)}, expected {hex(w)} ({c['why']})"
    nans = np.array([int(h, 16) for h in g["nan_inputs"]], dtype=np.uint32)
    out = oracle.round_bf16(nans.view(np.float32))
    widened = (out.astype(np.uint32) << 16).view(np.float32)
    assert np.all(np.isnan(widened))


def test_bf16_matches_torch_cast():
    import torch
    rng = np.random.default_rng(5)
    bits = rng.integers(0, 2 ** 32, size=1 << 20, dtype=np.uint64).astype(np.uint32)
    f = bits.view(np.float32)
    f = f[~np.isnan(f)]
    want = torch.from_numpy(f.copy()).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.round_bf16(f), want)


def test_widen_bf16_exact():
    bits = np.array([0x3f80, 0xc049, 0x0001, 0x7f7f, 0x8000], dtype=np.uint16)
    vals = oracle.widen_bf16(bits)
    assert vals[0] == 1.0
    assert vals[1] == -3.140625
    assert vals[2] == 2.0 ** -133
    assert vals[3] == (2 - 2.0 ** -7) * 2.0 ** 127
    assert vals[4] == 0.0 and np.signbit(vals[4])


# ---------------------------------------------------------------------------
# Index maps (placements) against the values printed on the pages and the
# "every shard covers each global index exactly once" invariant.
# ---------------------------------------------------------------------------

def test_printed_distribute_rows():
    with open(os.path.join(GOLDEN, "layout_examples.json")) as f:
        g = json.load(f)["distribute_rows"]
    A = np.array(g["global"])
    shards = oracle.split(A, g["P"], g["placement"]["dim"])
    for got, want in zip(shards, g["shards"]):
        assert np.array_equal(got, np.array(want))


def test_printed_shapes():
    with open(os.path.join(GOLDEN, "layout_examples.json")) as f:
        g = json.load(f)
    e = g["global_shape_from_local"]
    R, C = e["local_shape"][0] * e["P"], e["local_shape"][1]
    assert [R, C] == e["global_shape"]
    v = oracle.expected_views(R, C, C, oracle.SHARD, e["dim"], e["P"])
    assert all((r, c) == tuple(e["local_shape"]) for _, r, c, _, _, _ in v)
    for key in ("batch_split", "weight_column_split"):
        e = g[key]
        R, C = e["global_shape"]
        v = oracle.expected_views(R, C, C, oracle.SHARD, e["dim"], e["P"])
        assert all([r, c] == e["local_shape"] for _, r, c, _, _, _ in v)


@pytest.mark.parametrize("R,C", [(1, 1), (4, 4), (6, 10), (8, 3), (12, 12)])
def test_index_sets_cover_exactly_once(R, C):
    for dim in (0, 1, -1, -2):
        L = R if dim in (0, -2) else C
        for P in range(1, L + 1):
            if L % P:
                with pytest.raises(ValueError):
                    oracle.shard_index_sets(R, C, oracle.SHARD, dim, P)
                continue
            sets = oracle.shard_index_sets(R, C, oracle.SHARD, dim, P)
            count = {}
            for s in sets:
                for rc in s:
                    count[rc] = count.get(rc, 0) + 1
            assert len(count) == R * C and set(count.values()) == {1}
            # Closed form: shard i of dim d is [i*L/P, (i+1)*L/P).
            views = oracle.expected_views(R, C, C + 3, oracle.SHARD, dim, P)
            for i, (off, r, c, ld, r0, c0) in enumerate(views):
                if dim in (0, -2):
                    assert (r, c, r0, c0) == (R // P, C, i * R // P, 0)
                else:
                    assert (r, c, r0, c0) == (R, C // P, 0, i * C // P)
                assert off == r0 * (C + 3) + c0 and ld == C + 3
    for kind in (oracle.REPLICATE, oracle.PARTIAL):
        sets = oracle.shard_index_sets(R, C, kind, 0, 3)
        assert all(len(s) == R * C for s in sets)


# ---------------------------------------------------------------------------
# Comparison metrics.  Every tolerance verdict goes through rel_l2 and max_abs, so
# they are pinned to values worked out by hand from their definitions:
# rel_l2 = ||got - ref||_2 / ||ref||_2, max_abs = max |got - ref|.
# ---------------------------------------------------------------------------

def test_rel_l2_closed_forms():
    # one element off by d: |d| / ||ref||; ref (3, 4) has norm 5 exactly.
    assert oracle.rel_l2([3.0, 6.0], [3.0, 4.0]) == 0.4        # ||got||: 2/sqrt(45)
    assert oracle.rel_l2([3.0, 2.0], [3.0, 4.0]) == 0.4
    # no square roots: 0.16 would be (d / ||ref||)^2
    assert oracle.rel_l2([1.0, 2.0], [1.0, 1.0]) == pytest.approx(1 / np.sqrt(2), rel=1e-15)
    # argument order matters: the reference's norm is the denominator
    assert oracle.rel_l2([2.0], [1.0]) == 1.0
    assert oracle.rel_l2([1.0], [2.0]) == 0.5
    # a uniform relative error eps on every element gives exactly |eps|
    ref = np.random.default_rng(7).standard_normal((17, 33))
    for eps in (0.5, -0.25, 2.0 ** -10):
        assert oracle.rel_l2(ref * (1 + eps), ref) == pytest.approx(abs(eps), rel=1e-12)
    # zero reference: 0 when equal, infinite otherwise
    assert oracle.rel_l2([0.0, 0.0], [0.0, 0.0]) == 0.0
    assert oracle.rel_l2([3.0, 4.0], [0.0, 0.0]) == float("inf")
    # all elements count, in any layout (2-D here)
    assert oracle.rel_l2([[0.0, 3.0], [4.0, 5.0]], [[0.0, 3.0], [4.0, 0.0]]) == 1.0


def test_max_abs_closed_forms():
    assert oracle.max_abs([-5.0], [0.0]) == 5.0
    assert oracle.max_abs([0.0], [-5.0]) == 5.0
    # the largest magnitude, not the largest signed difference (that is 2)
    assert oracle.max_abs([0.0, -3.0, 2.0], [0.0, 0.0, 0.0]) == 3.0
    assert oracle.max_abs([[1.5, 1.0], [1.0, -7.0]], [[1.0, 1.0], [1.0, 1.0]]) == 8.0
    assert oracle.max_abs(np.zeros((0, 4)), np.zeros((0, 4))) == 0.0


def test_metrics_reject_shape_mismatch():
    # got - ref must not broadcast: a (N,) result against a (rows, N)
    # reference is a harness mistake, not a comparison.
    for f in (oracle.rel_l2, oracle.max_abs):
        with pytest.raises(ValueError):
            f(np.zeros(4), np.zeros((3, 4)))
        with pytest.raises(ValueError):
            f(np.zeros((4, 1)), np.zeros((4, 4)))
        with pytest.raises(ValueError):
            f(np.zeros((2, 3)), np.zeros((3, 2)))
