"""GPU parity at the full workload sizes, in the launch configuration the
throughput benchmark times.

The benchmark's Workload object is built as it is there (same shapes, same
seeded device-drawn inputs, same library calls), each op runs once, and the
outputs are checked on sampled token rows against the CPU oracle: every
output row depends only on its own input row and all of W, so the oracle
takes the sampled rows of X and the whole of W (copied to the host; the
oracle never sees a result of the HIP path).  Sampled rows: row 0, one
seeded row in every block of 256, and row M-1.

Bar (bf16 inputs, fp32 accumulation): rel L2 <= 1e-2 and
max abs <= 2e-2 sqrt(K) sigma_x sigma_w, on every checked output.
"""
import gc

import numpy as np
import pytest
import torch

import bench
import oracle
import synth
import tensor_linear_amd as tl
from gpu_util import bf16_tol

pytestmark = pytest.mark.gpu

RTOL_L2 = 1e-2


def _host64(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def _w_io(W: torch.Tensor) -> np.ndarray:
    """Stored [N, K] weight -> fp64 [K, N] (the pages' [in, out] formula)."""
    return np.ascontiguousarray(_host64(W).T)


def _check(name, got, ref, K, sw=synth.SIGMA_W):
    r, m = oracle.rel_l2(got, ref), oracle.max_abs(got, ref)
    tol = bf16_tol(K, synth.SIGMA_X, sw)
    print(f"{name}: rel_l2={r:.3e} max_abs={m:.3e} (tol {tol:.3e})", flush=True)
    assert np.all(np.isfinite(got)), f"{name}: non-finite output"
    assert r <= RTOL_L2, f"{name}: rel L2 {r:.3e}"
    assert m <= tol, f"{name}: max abs {m:.3e} > {tol:.3e}"


def _run(wl):
    for name, _, _, fn in wl.ops:
        print(f"  launch {name}", flush=True)
        fn()
    torch.cuda.synchronize()


def _free(wl):
    del wl
    gc.collect()
    torch.cuda.empty_cache()


@pytest.mark.parametrize("wid", [2, 3])
def test_prefill_workload_sampled_rows(wid):
    """Column GEMM, row GEMM partials and the shard fold (Llama-8B MLP shard,
    Llama-70B attention shard); the fused row layer against that fold."""
    print(f"workload {wid}", flush=True)
    wl = bench.Workload(wid, torch, tl, synth)
    _run(wl)
    P, sh = wl.P, wl.shape
    rows = synth.sample_rows(sh["M"], seed=77 + wid)

    # column: Y1 = X1 W1 (concatenated shards)
    X64 = _host64(wl.X1[rows])
    ref = oracle.column_parallel_linear(X64, _w_io(wl.W1), P)
    _check("column Y1", _host64(wl.Y1[rows]), ref, sh["K1"])

    # row: partials, then the fold
    X64 = _host64(wl.X2[rows])
    parts = oracle.row_partials(X64, _w_io(wl.W2), P)
    got_parts = _host64(wl.parts[:, rows])
    for i in range(P):
        _check(f"row partial {i}", got_parts[i], parts[i], sh["K2"] // P)
    _check("row fold Y2", _host64(wl.Y2[rows]), oracle.fold_f64(parts), sh["K2"])

    # the whole row layer through TP_ROW_FUSED (the fold in registers at
    # these shard K): bit for bit the fold of the partials above, all rows
    M, N = wl.Y2.shape
    Yf = torch.full((M, N), float("nan"), dtype=wl.Y2.dtype, device=wl.Y2.device)
    ws = torch.empty(tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, M, N, P), dtype=torch.uint8,
                     device=wl.Y2.device)
    print("  launch row layer TP_ROW_FUSED", flush=True)
    tl.tp_linear_row(wl.X2, wl.W2, Yf, P, tl.TP_ROW_FUSED, ws)
    torch.cuda.synchronize()
    assert torch.equal(Yf.view(torch.int16), wl.Y2.view(torch.int16))
    del Yf, ws
    _free(wl)


def test_decode_workload_all_rows():
    """Decode shapes (M = 16): skinny column GEMM and the row GEMM with the
    fold fused into its epilogue, all output rows."""
    wl = bench.Workload(4, torch, tl, synth)
    _run(wl)
    P, sh = wl.P, wl.shape
    ref = oracle.column_parallel_linear(_host64(wl.X1), _w_io(wl.W1), P)
    _check("decode column Y1", _host64(wl.Y1), ref, sh["hidden"])
    ref = oracle.row_parallel_linear(_host64(wl.X2), _w_io(wl.W2), P)
    _check("decode fused row Y2", _host64(wl.Y2), ref, sh["intermediate"])
    _free(wl)


def test_sequence_parallel_workload_sampled_rows():
    """Row GEMM partials, the reduce-scatter fold into P token slices, and the
    column GEMM that reads the slices back as one all-gathered tensor."""
    wl = bench.Workload(5, torch, tl, synth)
    _run(wl)
    P, sh = wl.P, wl.shape
    M, N, K, N3 = sh["M"], sh["N"], sh["K"], sh["N_next"]
    rows = synth.sample_rows(M, seed=82)

    X64 = _host64(wl.X1[rows])
    parts = oracle.row_partials(X64, _w_io(wl.W1), P)
    got_parts = _host64(wl.parts[:, rows])
    for i in range(P):
        _check(f"row partial {i}", got_parts[i], parts[i], K // P)

    # Token slice j holds rows [j*M/P, (j+1)*M/P) of the sum; with the
    # default slice stride the slices sit back to back in Y.
    s = M // P
    slices = wl.Y.view(P, s, N)
    got = np.stack([_host64(slices[m // s, m % s]) for m in rows])
    _check("reduce-scatter slices", got, oracle.fold_f64(parts), K)

    # TP_ROW_SCATTER in one call (the fold in registers at this shard K):
    # bit for bit the slices above, all rows
    Ys = torch.full_like(wl.Y, float("nan"))
    ws = torch.empty(tl.tp_row_workspace_bytes(tl.TP_ROW_SCATTER, M, N, P), dtype=torch.uint8,
                     device=wl.Y.device)
    print("  launch row layer TP_ROW_SCATTER", flush=True)
    tl.tp_linear_row(wl.X1, wl.W1, Ys, P, tl.TP_ROW_SCATTER, ws)
    torch.cuda.synchronize()
    assert torch.equal(Ys.view(torch.int16), wl.Y.view(torch.int16))
    del Ys, ws

    # The next column GEMM reads the gathered slices.  The oracle's input
    # is its own bf16 result of the row stage (fp32 partials, fp32 fold,
    # one rounding), never the device's.
    p32 = np.stack([p.astype(np.float32) for p in parts])
    y_bf16 = oracle.widen_bf16(oracle.round_bf16(oracle.fold_f32(p32)))
    ref = oracle.column_parallel_linear(y_bf16, _w_io(wl.W3), P)
    # the row-stage output has std ~ sqrt(K) sigma_w, the column stage's input
    sy = float(np.sqrt(np.mean(y_bf16 ** 2)))
    got = _host64(wl.Y3[rows])
    r, m = oracle.rel_l2(got, ref), oracle.max_abs(got, ref)
    tol = 2e-2 * np.sqrt(N) * sy * synth.SIGMA_W
    print(f"all-gathered column Y3: rel_l2={r:.3e} max_abs={m:.3e} (tol {tol:.3e})", flush=True)
    assert r <= RTOL_L2 and m <= tol
    _free(wl)


def _swiglu_bound(G, U, K, sw):
    """Per-element bar for silu(g) * u: the bf16 bar of each product,
    t = 2e-2 sqrt(K) sx sw, carried through the unit to first order, plus one
    bf16 rounding of the output (2^-8 |h|)."""
    t = bf16_tol(K, synth.SIGMA_X, sw)
    sig = 1.0 / (1.0 + np.exp(-G))
    dsilu = sig * (1.0 + G * (1.0 - sig))
    return t * (np.abs(dsilu * U) + np.abs(G * sig)) + 2.0 ** -8 * np.abs(G * sig * U)


def test_mlp_layer_workload_sampled_rows():
    """The Llama-8B MLP layer with its biases: the gate+up column GEMM with
    the Shard(0) bias and silu(gate) * up fused, the row GEMM on the gated
    output, and the fold with the Partial() bias added once."""
    wl = bench.Workload(6, torch, tl, synth)
    _run(wl)
    P, sh = wl.P, wl.shape
    H, I = sh["hidden"], sh["intermediate"]
    rows = synth.sample_rows(sh["M"], seed=86)

    G, U = oracle.column_parallel_gate_up(_host64(wl.X1[rows]), _w_io(wl.W1), _host64(wl.b1), P)
    ref = oracle.swiglu(G, U)
    got = _host64(wl.H[rows])
    r = oracle.rel_l2(got, ref)
    worst = float(np.max(np.abs(got - ref) / _swiglu_bound(G, U, H, synth.SIGMA_W)))
    print(f"gated column H: rel_l2={r:.3e} worst err/bound={worst:.3f}", flush=True)
    assert np.all(np.isfinite(got)) and r <= RTOL_L2 and worst <= 1.0

    # The row stage's oracle input is the oracle's own bf16 gated output.
    h_bf16 = oracle.widen_bf16(oracle.round_bf16(ref.astype(np.float32)))
    parts = oracle.row_partials(h_bf16, _w_io(wl.W2), P)
    yref = oracle.fold_f64(parts) + _host64(wl.b2)[None, :]
    sh_ = float(np.sqrt(np.mean(h_bf16 ** 2)))
    got = _host64(wl.Y2[rows])
    r, m = oracle.rel_l2(got, yref), oracle.max_abs(got, yref)
    tol = 2e-2 * np.sqrt(I) * sh_ * synth.SIGMA_W
    print(f"row fold + bias Y2: rel_l2={r:.3e} max_abs={m:.3e} (tol {tol:.3e})", flush=True)
    assert r <= RTOL_L2 and m <= tol
    _free(wl)


def test_sequence_parallel_separate_slices_sampled_rows():
    """The sequence-parallel round trip with the token slices in P separate
    allocations: the reduce-scatter writes them, the next column GEMM reads
    them in place."""
    wl = bench.Workload(7, torch, tl, synth)
    _run(wl)
    P, sh = wl.P, wl.shape
    M, N, K = sh["M"], sh["N"], sh["K"]
    rows = synth.sample_rows(M, seed=87)
    parts = oracle.row_partials(_host64(wl.X1[rows]), _w_io(wl.W1), P)
    s = M // P
    got = np.stack([_host64(wl.slices[m // s][m % s]) for m in rows])
    _check("reduce-scatter slice allocations", got, oracle.fold_f64(parts), K)
    p32 = np.stack([p.astype(np.float32) for p in parts])
    y_bf16 = oracle.widen_bf16(oracle.round_bf16(oracle.fold_f32(p32)))
    ref = oracle.column_parallel_linear(y_bf16, _w_io(wl.W3), P)
    sy = float(np.sqrt(np.mean(y_bf16 ** 2)))
    got = _host64(wl.Y3[rows])
    r, m = oracle.rel_l2(got, ref), oracle.max_abs(got, ref)
    tol = 2e-2 * np.sqrt(N) * sy * synth.SIGMA_W
    print(f"column on slice allocations Y3: rel_l2={r:.3e} max_abs={m:.3e} (tol {tol:.3e})",
          flush=True)
    assert r <= RTOL_L2 and m <= tol
    _free(wl)


def test_embedding_workload_all_tokens():
    """The Llama-8B embedding sharded on its feature dim, every token: a
    lookup copies bits, so the output equals the oracle's bit for bit."""
    wl = bench.Workload(8, torch, tl, synth)
    _run(wl)
    P = wl.P
    E = np.concatenate([t.cpu().view(torch.int16).numpy().view(np.uint16) for t in wl.E], axis=1)
    ids = wl.ids.cpu().numpy()
    ref = oracle.embedding_parallel(ids, E, P)
    got = wl.Y1.cpu().view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(got, ref)
    _free(wl)
