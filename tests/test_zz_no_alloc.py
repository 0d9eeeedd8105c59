"""tp_linear_row_noalloc (the row-parallel Linear for callers that cannot
allocate) against tp_linear_row with a caller workspace: the same kernels, so
the outputs must be equal bit for bit.  Two calls in a row, the second with a
smaller input, for every mode that uses the workspace, bf16 and fp32; calls
whose fold runs inside the GEMM at sizes whose partials would not fit the
fixed array; captured in a HIP graph and replayed; and the rejection of a
call whose partials would not fit."""
import numpy as np
import pytest
import torch

import tensor_linear_amd as tl
from gpu_util import DEV, bits, workspace

pytestmark = pytest.mark.gpu

# (M, K, N, P): the first call's partials fill 16 MiB of the 32 MiB array,
# the second is smaller and ragged
SHAPES = [(512, 4096, 1024, 8), (72, 600, 200, 4)]


def _inputs(M, K, N, dtype, seed):
    gen = torch.Generator(device=DEV)
    gen.manual_seed(seed)
    X = torch.randn((M, K), generator=gen, device=DEV).to(dtype)
    W = (torch.randn((N, K), generator=gen, device=DEV) * 0.02).to(dtype)
    return X, W


@pytest.mark.parametrize("dtype", [torch.bfloat16, torch.float32])
@pytest.mark.parametrize("mode", [tl.TP_ROW_SUM, tl.TP_ROW_FUSED, tl.TP_ROW_SCATTER,
                                  tl.TP_ROW_PARTIAL])
def test_noalloc_equals_workspace_call(dtype, mode):
    for i, (M, K, N, P) in enumerate(SHAPES):
        print(f"noalloc mode={mode} dtype={dtype} M={M} K={K} N={N} P={P}", flush=True)
        assert tl.tp_row_workspace_bytes(mode, M, N, P) <= tl.TP_NOALLOC_SCRATCH_BYTES
        X, W = _inputs(M, K, N, dtype, 300 + i)
        if mode == tl.TP_ROW_PARTIAL:
            ref = torch.empty((P, M, N), dtype=torch.float32, device=DEV)
            got = torch.full((P, M, N), float("nan"), dtype=torch.float32, device=DEV)
        else:
            ref = torch.empty((M, N), dtype=dtype, device=DEV)
            got = torch.full((M, N), float("nan"), dtype=dtype, device=DEV)
        tl.tp_linear_row(X, W, ref, P, mode, workspace(mode, M, N, P))
        tl.tp_linear_row_noalloc(X, W, got, P, mode)
        torch.cuda.synchronize()
        assert np.array_equal(bits(got), bits(ref)), f"call {i}"


@pytest.mark.parametrize("M,K,N,P,mode", [
    (2048, 8192, 1024, 8, tl.TP_ROW_FUSED),     # prefill, the fold in registers
    (2048, 8192, 1024, 8, tl.TP_ROW_SCATTER),   # the same, into 256-row token slices
    (48, 512, 32768, 8, tl.TP_ROW_FUSED),       # decode, the fused skinny fold
])
def test_noalloc_fused_paths_need_no_workspace(M, K, N, P, mode):
    # 48 or 64 MiB of fp32 partials would not fit the array, but these calls fold
    # inside the GEMM and use none of it
    print(f"noalloc fused M={M} K={K} N={N} P={P} mode={mode}", flush=True)
    assert tl.tp_row_workspace_bytes(mode, M, N, P) > tl.TP_NOALLOC_SCRATCH_BYTES
    X, W = _inputs(M, K, N, torch.bfloat16, 11)
    ref = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    got = torch.full((M, N), float("nan"), dtype=torch.bfloat16, device=DEV)
    tl.tp_linear_row(X, W, ref, P, mode, workspace(mode, M, N, P))
    tl.tp_linear_row_noalloc(X, W, got, P, mode)
    torch.cuda.synchronize()
    assert np.array_equal(bits(got), bits(ref))


@pytest.mark.parametrize("M,K,N,P,mode", [
    (512, 4096, 1024, 8, tl.TP_ROW_SUM),        # partials in the fixed array, then the fold
    (2048, 8192, 1024, 8, tl.TP_ROW_FUSED),     # the fold in registers, no array
])
def test_noalloc_under_graph_capture(M, K, N, P, mode):
    # the callers the entry point is for: a captured step, replayed with new
    # inputs written eagerly between replays, each replay bitwise equal to
    # the workspace call run eagerly (the first call, which looks up the
    # array's address, runs before the capture, on a side stream)
    print(f"noalloc graph M={M} K={K} N={N} P={P} mode={mode}", flush=True)
    gen = torch.Generator(device=DEV)
    gen.manual_seed(21)
    X = torch.randn((M, K), generator=gen, device=DEV).to(torch.bfloat16)
    W = (torch.randn((N, K), generator=gen, device=DEV) * 0.02).to(torch.bfloat16)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        tl.tp_linear_row_noalloc(X, W, Y, P, mode)
    torch.cuda.current_stream().wait_stream(side)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        tl.tp_linear_row_noalloc(X, W, Y, P, mode)
    torch.cuda.synchronize()
    ws = workspace(mode, M, N, P)
    for r in range(3):
        X.copy_(torch.randn((M, K), generator=gen, device=DEV).to(torch.bfloat16))
        graph.replay()
        torch.cuda.synchronize()
        ref = torch.empty_like(Y)
        tl.tp_linear_row(X, W, ref, P, mode, ws)
        torch.cuda.synchronize()
        assert np.array_equal(bits(Y), bits(ref)), f"replay {r}"


def test_noalloc_rejects_oversized_workspace():
    M, K, N, P = 2048, 64, 1024, 8      # 64 MiB of partials
    X, W = _inputs(M, K, N, torch.bfloat16, 7)
    Y = torch.empty((M, N), dtype=torch.bfloat16, device=DEV)
    with pytest.raises(tl.TPError) as e:
        tl.tp_linear_row_noalloc(X, W, Y, P, tl.TP_ROW_SUM)
    assert e.value.status == tl.TP_ERR_WORKSPACE
