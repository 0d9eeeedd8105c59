"""CPU oracle for the tensor-parallel Linear Y = X W.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check in
__graft_entry__.py and the CPU-baseline leg of bench.py may import this
package.  It shares no code with the HIP library in tensor_linear_amd/ and
imports nothing from it.

Every step below is the plain definition from the pages, slow and explicit:

  * "模型并行" (wineandchord.com), section "Tensor Parallel":
      column parallel: W = [W_1, ..., W_P] split on the output dim, Y_i = X W_i;
      row parallel:    X = [X_1 .. X_P], W = [W_1; ..; W_P] split on the
                       input dim, Y = sum_i X_i W_i;
    section "Tensor-parallel 线性层": the weight is in the [in,out]
    orientation, the split needs the dim to divide evenly, the column results
    are concatenated along the output dim, the row results are summed, and
    every shard covers each global index exactly once.
  * "DTensor API 文档" (MindSpore hyper-parallel), sections "distribute_tensor"
    and "放置策略类型": Shard(d) gives each device its slice of dim d,
    Replicate() a full copy, Partial() a part that still has to be summed.
  * "3D 并行的实现：TP / PP / DP 各占几行" (nanotron), section "5.1 TP" and
    "模型并行", "Sequence Parallel": the row result may instead be
    reduce-scattered over tokens and later all-gathered.

Readings where the pages leave a point open:
  * the P partial results are summed in ascending shard order, left to right;
  * the reduce-scatter splits the token dim (dim 0) into P equal row blocks,
    block j going to shard j;
  * bf16 rounding is round-to-nearest-even;
  * the row bias (Partial()) enters the reduced sum once, after the last shard;
  * a fused gate+up column weight holds, per shard, its gate features first
    and then its up features; the gated unit is silu(gate) * up;
  * an embedding id outside [0, V) gives a zero output row.

Arithmetic: inputs (fp32 values or bf16 bit patterns) are widened exactly to
fp64 and the products are summed in fp64 by orc_dense (oracle.c), k ascending.
The fp32 fold and the bf16 rounding used as bit-exact references are in
oracle.c as well.
"""
import ctypes
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def _load():
    global _lib
    if _lib is not None:
        return _lib
    path = os.path.join(_HERE, "liboracle.so")
    if not os.path.exists(path) or (
            os.path.getmtime(path) < os.path.getmtime(os.path.join(_HERE, "oracle.c"))):
        _build.build()
    lib = ctypes.CDLL(path)
    i64, dptr, fptr = ctypes.c_int64, ctypes.c_void_p, ctypes.c_void_p
    lib.orc_dense.argtypes = [dptr, i64, dptr, i64, dptr, i64, i64, i64, i64]
    lib.orc_dense.restype = None
    lib.orc_fold_f32.argtypes = [fptr, i64, i64, i64, i64, ctypes.c_int32, fptr, fptr, i64]
    lib.orc_fold_f32.restype = None
    lib.orc_round_bf16.argtypes = [fptr, ctypes.c_void_p, i64]
    lib.orc_round_bf16.restype = None
    lib.orc_num_threads.argtypes = []
    lib.orc_num_threads.restype = ctypes.c_int
    _lib = lib
    return lib


def num_threads() -> int:
    """Threads the oracle's OpenMP loops run on."""
    return int(_load().orc_num_threads())


# ---------------------------------------------------------------------------
# Exact widening of the input formats to fp64.
# ---------------------------------------------------------------------------

def widen_bf16(bits: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> fp64.  A bf16 value is the fp32 value
    whose upper 16 bits are the pattern and whose lower 16 bits are zero,
    so the widening is exact."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def widen_f32(a: np.ndarray) -> np.ndarray:
    return np.asarray(a, dtype=np.float32).astype(np.float64)


# ---------------------------------------------------------------------------
# Dense product.
# ---------------------------------------------------------------------------

def dense(X: np.ndarray, W_io: np.ndarray) -> np.ndarray:
    """Y = X W, fp64, with W in [in,out] orientation ("模型并行",
    "Tensor Parallel", Y = XW).  Triple loop in oracle.c, k ascending."""
    X = np.ascontiguousarray(X, dtype=np.float64)
    W_io = np.ascontiguousarray(W_io, dtype=np.float64)
    if X.ndim != 2 or W_io.ndim != 2 or X.shape[1] != W_io.shape[0]:
        raise ValueError(f"dense: shapes {X.shape} x {W_io.shape}")
    M, K = X.shape
    N = W_io.shape[1]
    Y = np.empty((M, N), dtype=np.float64)
    if M and N:
        _load().orc_dense(X.ctypes.data, K, W_io.ctypes.data, N,
                          Y.ctypes.data, N, M, K, N)
    return Y


# ---------------------------------------------------------------------------
# Explicit split into P shards ("模型并行", "Tensor-parallel 线性层":
# the split dim must divide evenly; shard i is the i-th contiguous chunk).
# ---------------------------------------------------------------------------

def split(A: np.ndarray, P: int, dim: int) -> list:
    """Copies of the P equal contiguous chunks of A along dim."""
    if P < 1:
        raise ValueError("P must be >= 1")
    L = A.shape[dim]
    if L % P != 0:
        raise ValueError(f"dim {dim} of size {L} does not split into {P} equal shards")
    s = L // P
    out = []
    for i in range(P):
        idx = [slice(None)] * A.ndim
        idx[dim] = slice(i * s, (i + 1) * s)
        out.append(np.array(A[tuple(idx)], copy=True))
    return out


# ---------------------------------------------------------------------------
# Column parallel and row parallel.
# ---------------------------------------------------------------------------

def column_shards(X: np.ndarray, W_io: np.ndarray, P: int) -> list:
    """Y_i = X W_i for the P output-dim shards W_i of W ("Column parallel")."""
    return [dense(X, Wi) for Wi in split(W_io, P, 1)]


def column_parallel_linear(X: np.ndarray, W_io: np.ndarray, P: int) -> np.ndarray:
    """Concatenation of the Y_i along the output dim (the full tensor the
    page compares with the dense product)."""
    return np.concatenate(column_shards(X, W_io, P), axis=1)


def row_partials(X: np.ndarray, W_io: np.ndarray, P: int) -> list:
    """The P partial products X_i W_i, X split on its last dim and W on its
    first ("Row parallel"), each exact in fp64."""
    xs = split(X, P, 1)
    ws = split(W_io, P, 0)
    return [dense(xi, wi) for xi, wi in zip(xs, ws)]


def fold_f64(parts: list) -> np.ndarray:
    """Sum of the parts in ascending shard order, fp64."""
    acc = np.array(parts[0], dtype=np.float64, copy=True)
    for p in parts[1:]:
        acc = acc + p
    return acc


def row_parallel_linear(X: np.ndarray, W_io: np.ndarray, P: int) -> np.ndarray:
    """Y = sum_i X_i W_i (fp64, ascending shard order)."""
    return fold_f64(row_partials(X, W_io, P))


# ---------------------------------------------------------------------------
# The fp32 shard fold and bf16 rounding (bit-exact references).
# ---------------------------------------------------------------------------

def fold_f32(partials: np.ndarray, bias=None) -> np.ndarray:
    """partials: fp32 [P, M, N].  Returns fp32 [M, N] =
    ((p_0 + p_1) + ...) + p_{P-1}, one fp32 add at a time (oracle.c).
    bias: None or fp32 [N], the Partial() row bias of the whole layer, added
    once after the last shard (one more fp32 add)."""
    p = np.ascontiguousarray(partials, dtype=np.float32)
    if p.ndim != 3:
        raise ValueError("partials must be [P, M, N]")
    P, M, N = p.shape
    out = np.empty((M, N), dtype=np.float32)
    b = None
    if bias is not None:
        b = np.ascontiguousarray(bias, dtype=np.float32)
        if b.shape != (N,):
            raise ValueError("bias must be [N]")
    if M and N:
        _load().orc_fold_f32(p.ctypes.data, M * N, N, M, N, P,
                             None if b is None else b.ctypes.data, out.ctypes.data, N)
    return out


def round_bf16(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns (uint16), round to nearest even (oracle.c)."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    out = np.empty(f.shape, dtype=np.uint16)
    if f.size:
        _load().orc_round_bf16(f.ctypes.data, out.ctypes.data, f.size)
    return out


# ---------------------------------------------------------------------------
# Reduce-scatter over tokens and the all-gather that undoes it.
# ---------------------------------------------------------------------------

def reduce_scatter_rows(parts: list, P: int, fold=fold_f64) -> list:
    """Sum the partial results, then keep token (row) block j for shard j."""
    return split(fold(parts), P, 0)


def all_gather_rows(slices: list) -> np.ndarray:
    """Concatenate the token slices back along dim 0 (Shard(0) -> Replicate)."""
    return np.concatenate(slices, axis=0)


# ---------------------------------------------------------------------------
# Steps next to the Linear: the bias, the gated activation of the fused
# gate+up column layer, the column layer fed by token slices, and the
# embedding sharded on its feature dim.
# ---------------------------------------------------------------------------

def column_parallel_linear_bias(X: np.ndarray, W_io: np.ndarray, b, P: int) -> np.ndarray:
    """Y_i = X W_i + b_i, concatenated.  The column bias is Shard(0) ("Linear
    实现解析", tp_shard_type table, row "col"): shard i holds the bias of its
    own output features, split exactly like W's output dim."""
    bs = split(np.asarray(b, dtype=np.float64), P, 0)
    ys = column_shards(X, W_io, P)
    return np.concatenate([y + bi[None, :] for y, bi in zip(ys, bs)], axis=1)


def silu(g: np.ndarray) -> np.ndarray:
    """silu(g) = g * sigmoid(g) = g / (1 + exp(-g)), fp64.  (For g below about
    -709, exp(-g) overflows to inf and the quotient is the correct limit, a
    signed zero.)"""
    g = np.asarray(g, dtype=np.float64)
    with np.errstate(over="ignore"):
        return g / (1.0 + np.exp(-g))


def swiglu(g: np.ndarray, u: np.ndarray) -> np.ndarray:
    """The gated unit of the Llama MLP: silu(gate) * up, fp64."""
    return silu(g) * np.asarray(u, dtype=np.float64)


def column_parallel_gate_up(X: np.ndarray, W_io: np.ndarray, b, P: int):
    """The gate and up pre-activations of a fused gate+up column layer.

    W_io [K, 2I] is split into P output shards (Column parallel).  Reading
    of the fused layout: shard i's 2I/P output features hold its I/P gate
    features first, then its I/P up features, so gate_i and up_i of the same
    hidden units live on the same shard.  b (None or [2I]) is split the same
    way.  Returns (G, U), each [M, I], shard i's part at columns
    [i I/P, (i+1) I/P)."""
    ys = column_shards(X, W_io, P)
    if b is not None:
        bs = split(np.asarray(b, dtype=np.float64), P, 0)
        ys = [y + bi[None, :] for y, bi in zip(ys, bs)]
    gs, us = [], []
    for y in ys:
        g, u = split(y, 2, 1)
        gs.append(g)
        us.append(u)
    return np.concatenate(gs, axis=1), np.concatenate(us, axis=1)


def column_parallel_swiglu(X: np.ndarray, W_io: np.ndarray, b, P: int) -> np.ndarray:
    """H = silu(G) * U over the shards of a fused gate+up column layer
    (see column_parallel_gate_up for the layout), [M, I]."""
    G, U = column_parallel_gate_up(X, W_io, b, P)
    return swiglu(G, U)


def row_parallel_linear_bias(X: np.ndarray, W_io: np.ndarray, b, P: int) -> np.ndarray:
    """Y = sum_i X_i W_i + b.  The row bias is Partial() ("Linear 实现解析",
    tp_shard_type table, row "row"): its parts sum to the layer's bias, so
    the bias enters the reduced output once, added after the shard sum."""
    return row_parallel_linear(X, W_io, P) + np.asarray(b, dtype=np.float64)[None, :]


def column_parallel_linear_gathered(slices: list, W_io: np.ndarray, P: int) -> np.ndarray:
    """The column layer of the sequence-parallel layout: the P token slices
    are all-gathered (Shard(0) -> Replicate) into the full X, which then
    goes through the column-parallel product (nanotron "5.1 TP", column
    REDUCE_SCATTER mode: all_gather(x) before F.linear)."""
    return column_parallel_linear(all_gather_rows(slices), W_io, P)


def embedding_parallel(ids, E: np.ndarray, P: int) -> np.ndarray:
    """EmbeddingWithReplicateOutput ("Module 并行：实现 DP/TP/CP/PP 组合",
    section "DP / TP / CP / PP 并行实现", "Tensor Parallel": the embedding
    weight is Shard(1) on embedding_dim, the token ids are Replicate, and the
    output is all-gathered back to Replicate).

    E [V, D] is split into P feature shards E_i [V, D/P] (explicit copies);
    shard i looks up its rows, Y_i[t] = E_i[ids[t]], and the Y_i are
    concatenated along the feature dim.  Reading for an id outside [0, V)
    (the pages do not say): its output row is zero."""
    ids = np.asarray(ids, dtype=np.int64)
    V = E.shape[0]
    outs = []
    for Ei in split(np.asarray(E), P, 1):
        Yi = np.zeros((ids.shape[0], Ei.shape[1]), dtype=Ei.dtype)
        for t in range(ids.shape[0]):
            v = int(ids[t])
            if 0 <= v < V:
                Yi[t] = Ei[v]
        outs.append(Yi)
    return np.concatenate(outs, axis=1)


# ---------------------------------------------------------------------------
# Placements as integer index maps.
# ---------------------------------------------------------------------------

REPLICATE, SHARD, PARTIAL = 0, 1, 2


def shard_index_sets(rows: int, cols: int, kind: int, dim: int, P: int) -> list:
    """For each of the P shards, the set of global (r, c) indices it holds.

    Shard(dim): the tensor is tagged with its flat global index and split
    with the same explicit split as the data (`split`); each shard holds the
    indices that land in its chunk.  Replicate() and Partial(): every shard
    holds the full index set (for Partial, a full-shape part of the sum).
    dim may be negative (counted from the last of the 2 dims).
    """
    tags = np.arange(rows * cols, dtype=np.int64).reshape(rows, cols)
    if kind == SHARD:
        d = dim + 2 if dim < 0 else dim
        if d not in (0, 1):
            raise ValueError("dim out of range for a 2-D tensor")
        chunks = split(tags, P, d)
    elif kind in (REPLICATE, PARTIAL):
        if P < 1:
            raise ValueError("P must be >= 1")
        chunks = [tags.copy() for _ in range(P)]
    else:
        raise ValueError("unknown placement kind")
    out = []
    for ch in chunks:
        flat = ch.reshape(-1)
        out.append(set(zip((flat // cols).tolist(), (flat % cols).tolist())))
    return out


def expected_views(rows: int, cols: int, ld: int, kind: int, dim: int, P: int) -> list:
    """The rectangle each shard's index set spans, as (elem_offset, rows,
    cols, ld, row0, col0) with elem_offset = row0 * ld + col0 in a row-major
    buffer of leading dimension ld.  For Partial, part i is a separate
    full-shape buffer placed after the first i parts: elem_offset = i*rows*ld.
    Raises if a shard's set is not a full rectangle."""
    sets = shard_index_sets(rows, cols, kind, dim, P)
    views = []
    for i, s in enumerate(sets):
        if not s:
            views.append((0, 0, 0, ld, 0, 0))
            continue
        rs = sorted({r for r, _ in s})
        cs = sorted({c for _, c in s})
        if len(rs) * len(cs) != len(s) or rs != list(range(rs[0], rs[-1] + 1)) \
                or cs != list(range(cs[0], cs[-1] + 1)):
            raise AssertionError("shard index set is not a rectangle")
        off = rs[0] * ld + cs[0]
        if kind == PARTIAL:
            off = i * rows * ld
        views.append((off, len(rs), len(cs), ld, rs[0], cs[0]))
    return views


# ---------------------------------------------------------------------------
# Comparison metrics behind every tolerance bar (the page "模型并行",
# section "Tensor-parallel 线性层", compares the sharded result with the dense
# product element by element).
# ---------------------------------------------------------------------------

def _pair(got, ref):
    g = np.asarray(got, dtype=np.float64)
    r = np.asarray(ref, dtype=np.float64)
    if g.shape != r.shape:
        raise ValueError(f"shape mismatch: got {g.shape}, ref {r.shape}")
    return g, r


def rel_l2(got: np.ndarray, ref: np.ndarray) -> float:
    """||got - ref||_2 / ||ref||_2 in fp64 over all elements.  A zero ref
    gives 0 when got equals it and +inf otherwise.  Shapes must match."""
    g, r = _pair(got, ref)
    den = float(np.sqrt(np.sum(r * r)))
    num = float(np.sqrt(np.sum((g - r) ** 2)))
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return num / den


def max_abs(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| in fp64 (0 for empty arrays).  Shapes must match."""
    g, r = _pair(got, ref)
    if g.size == 0:
        return 0.0
    return float(np.max(np.abs(g - r)))
