"""The library's launches captured in a HIP graph (torch.cuda.CUDAGraph):
every entry point only queues kernels on the caller's stream -- no
allocation, no memset node, no host synchronisation -- so a captured step
replays correctly.  Each graph is replayed several times with new inputs
written eagerly between the replays, and every replay is compared bit for
bit with the same calls run eagerly."""
import pytest
import torch

import tensor_linear_amd as tl
from gpu_util import DEV, workspace

pytestmark = pytest.mark.gpu


def _rand(gen, shape, scale=1.0):
    return (torch.randn(shape, generator=gen, device=DEV) * scale).to(torch.bfloat16)


def _capture(fn):
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()                                     # warm-up on a side stream
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        fn()
    torch.cuda.synchronize()
    return graph


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a.view(torch.int32),
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b.view(torch.int32))


def test_graph_decode_step():
    # decode: column GEMM, then the row GEMM with the fold and bias fused
    M, H, I, P = 16, 2048, 4096, 8
    gen = torch.Generator(device=DEV)
    gen.manual_seed(1)
    X, W1, W2 = _rand(gen, (M, H)), _rand(gen, (I, H), 0.02), _rand(gen, (H, I), 0.02)
    b2 = _rand(gen, (H,), 0.02)
    Y1 = torch.empty((M, I), dtype=torch.bfloat16, device=DEV)
    Y2 = torch.empty((M, H), dtype=torch.bfloat16, device=DEV)
    ws = workspace(tl.TP_ROW_FUSED, M, H, P)

    def step(x, y1, y2):
        tl.tp_linear_column(x, W1, y1, P)
        tl.tp_linear_row_ex(y1, W2, y2, P, tl.TP_ROW_FUSED, ws, bias=b2)

    graph = _capture(lambda: step(X, Y1, Y2))
    for r in range(4):
        X.copy_(_rand(gen, (M, H)))              # eager work between replays
        graph.replay()
        torch.cuda.synchronize()
        E1, E2 = torch.empty_like(Y1), torch.empty_like(Y2)
        step(X, E1, E2)
        torch.cuda.synchronize()
        assert _same(Y1, E1) and _same(Y2, E2), f"replay {r}"


def test_graph_prefill_row_and_scatter():
    # tile GEMM partials, fold with bias into slice allocations, column GEMM
    # with the gated unit reading the slices
    M, K, N, P = 512, 1024, 1024, 4
    gen = torch.Generator(device=DEV)
    gen.manual_seed(2)
    X, W = _rand(gen, (M, K)), _rand(gen, (N, K), 0.02)
    Wgu, bgu, b = _rand(gen, (2 * 512, N), 0.02), _rand(gen, (2 * 512,), 0.02), _rand(gen, (N,), 0.02)
    parts = torch.empty((P, M, N), dtype=torch.float32, device=DEV)
    slices = [torch.empty((M // P, N), dtype=torch.bfloat16, device=DEV) for _ in range(P)]
    H = torch.empty((M, 512), dtype=torch.bfloat16, device=DEV)

    def step(x, pt, sl, h):
        tl.tp_linear_row(x, W, pt, P, tl.TP_ROW_PARTIAL)
        tl.tp_shard_reduce_ex(pt, None, P, scatter=1, bias=b, y_slices=sl)
        tl.tp_linear_column_ex(None, Wgu, h, P, bias=bgu, act=tl.TP_ACT_SWIGLU, x_slices=sl)

    graph = _capture(lambda: step(X, parts, slices, H))
    for r in range(3):
        X.copy_(_rand(gen, (M, K)))
        graph.replay()
        torch.cuda.synchronize()
        ep = torch.empty_like(parts)
        es = [torch.empty_like(t) for t in slices]
        eh = torch.empty_like(H)
        step(X, ep, es, eh)
        torch.cuda.synchronize()
        assert _same(parts, ep), f"replay {r}: partials"
        assert all(_same(a, e) for a, e in zip(slices, es)), f"replay {r}: slices"
        assert _same(H, eh), f"replay {r}: gated column"


def test_graph_embedding():
    V, D, T, P = 5000, 1024, 256, 8
    gen = torch.Generator(device=DEV)
    gen.manual_seed(3)
    shards = [_rand(gen, (V, D // P)) for _ in range(P)]
    ids = torch.randint(0, V, (T,), generator=gen, device=DEV, dtype=torch.int64)
    Y = torch.empty((T, D), dtype=torch.bfloat16, device=DEV)
    graph = _capture(lambda: tl.tp_embedding(ids, Y, P, e_shards=shards))
    for r in range(3):
        ids.copy_(torch.randint(0, V, (T,), generator=gen, device=DEV, dtype=torch.int64))
        graph.replay()
        torch.cuda.synchronize()
        E = torch.empty_like(Y)
        tl.tp_embedding(ids, E, P, e_shards=shards)
        torch.cuda.synchronize()
        assert _same(Y, E), f"replay {r}"
        assert _same(Y[:, :D // P], shards[0][ids]), f"replay {r}: against torch indexing"
