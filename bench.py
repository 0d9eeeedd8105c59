"""Throughput of the tensor-parallel Linear hot path on one MI355X.

A step is one pass of the path over one batch of synthetic input.  The
default workload is the Llama-8B MLP tensor-parallel shard: M = 4096 tokens,
hidden 4096, intermediate 14336, P = 8 shards resident on one GPU:
  fc1  column-parallel  X [4096, 4096]  x W1 [28672, 4096]^T -> Y1 [4096, 28672]
  fc2  row-parallel     X2 [4096, 14336] x W2 [4096, 14336]^T -> 8 fp32 partials
  fold ascending-shard sum of the 8 partials -> Y2 [4096, 4096] bf16
(tp_linear_column, tp_linear_row with TP_ROW_PARTIAL, tp_shard_reduce: the
same kernels TP_ROW_SUM runs, called separately so each is timed).

Prints ONE JSON line.  `value` is the step's GEMM TFLOP/s; `roofline` is for
the dominant kernel (the fc1 column GEMM, MFMA-bound), its time measured with
HIP events on the stream it runs on; `cpu_baseline` times the CPU oracle on a
bounded sample of the same workload; `context` holds figures taken outside the
timed step (each GEMM's shards launched alone, in turn, at their real shape, a plain device copy,
the shader clock while each GEMM runs and the roofline fraction at that clock:
the chip lowers its clock under sustained matrix-core load; and the platform's
own GEMM / gather on the same inputs, timed the same way).

Other workloads (--workload): 3 Llama-70B attention shard, 4 decode, 5
sequence-parallel round trip, 6 the Llama-8B MLP layer with its column and row
biases and the gated unit fused into the gate+up column GEMM (the row GEMM
reads the gated output), 7 the sequence-parallel round trip with the token
slices in P separate allocations (reduce-scatter writes them, the next column
GEMM reads them in place), 8 the Llama-8B token embedding sharded on its
feature dim (P shard tables in separate allocations, all-gathered output, a new
batch of token ids every step; its one-kernel steps are timed as a replay of
them captured in a HIP graph).

  python bench.py [--steps K] [--warmup W] [--gpus 1] [--workload 2..8]
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "TFLOP/s and % bf16 MFMA peak, TP column/row Linear shard GEMM; reduce GB/s"
PEAK_BF16_TFLOPS = 2516.6   # 256 CU x 2.4 GHz x 4096 flop/clk/CU, dense
PEAK_HBM_GBPS = 8000.0
PEAK_CLOCK_GHZ = 2.4        # the clock the bf16 peak assumes


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=50)
    ap.add_argument("--workload", type=int, default=2, choices=[2, 3, 4, 5, 6, 7, 8])
    ap.add_argument("--cpu-rows", type=int, default=3072,
                    help="rows of X the CPU oracle baseline computes")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-platform-reference", dest="platform_reference", action="store_false",
                    help="skip timing the platform's own GEMM / gather on the same inputs")
    ap.add_argument("--copy-calibration", type=int, default=0, metavar="MIB",
                    help="first run 3 device-to-device copies of this many MiB (a plain copy "
                         "of known size, to scale hardware byte counters)")
    return ap.parse_args()


class Workload:
    """Device buffers and the step for one workload."""

    def __init__(self, wid, torch, tl, synth):
        self.wid, self.torch, self.tl = wid, torch, tl
        dev = "cuda:0"
        P = 8
        self.P = P
        sx, sw = synth.SIGMA_X, synth.SIGMA_W
        nb = lambda g, t, shape, s: synth.device_normal_bf16(synth.seed_for(wid, g, t), shape, s, dev)
        bf = torch.bfloat16
        if wid in (2, 3):
            M, K1, N1, K2, N2 = {2: (4096, 4096, 28672, 14336, 4096),
                                 3: (8192, 8192, 10240, 8192, 8192)}[wid]
            self.X1, self.W1 = nb(0, 0, (M, K1), sx), nb(0, 1, (N1, K1), sw)
            self.X2, self.W2 = nb(1, 0, (M, K2), sx), nb(1, 1, (N2, K2), sw)
            self.Y1 = torch.empty((M, N1), dtype=bf, device=dev)
            self.parts = torch.empty((P, M, N2), dtype=torch.float32, device=dev)
            self.Y2 = torch.empty((M, N2), dtype=bf, device=dev)
            self.ops = [
                ("column_gemm", 2.0 * M * N1 * K1, None,
                 lambda: tl.tp_linear_column(self.X1, self.W1, self.Y1, P)),
                ("row_gemm", 2.0 * M * N2 * K2, None,
                 lambda: tl.tp_linear_row(self.X2, self.W2, self.parts, P, tl.TP_ROW_PARTIAL)),
                ("shard_fold", 0.0, P * M * N2 * 4 + M * N2 * 2,
                 lambda: tl.tp_shard_reduce(self.parts, self.Y2, P)),
            ]
            self.name = {2: "Llama-8B MLP TP shard: M=4096, hidden 4096, intermediate 14336, "
                            "P=8; fc1 column 4096->28672, fc2 row 14336->4096 + shard fold",
                         3: "Llama-70B attention TP shard: M=8192, hidden 8192, P=8; QKV column "
                            "8192->10240, O row 8192->8192 + shard fold"}[wid]
            self.shape = dict(M=M, K1=K1, N1=N1, K2=K2, N2=N2, P=P)
        elif wid == 4:
            M, H, I = 16, 8192, 28672
            self.X1, self.W1 = nb(0, 0, (M, H), sx), nb(0, 1, (I, H), sw)
            self.X2, self.W2 = nb(1, 0, (M, I), sx), nb(1, 1, (H, I), sw)
            self.Y1 = torch.empty((M, I), dtype=bf, device=dev)
            self.Y2 = torch.empty((M, H), dtype=bf, device=dev)
            nbytes = tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, M, H, P)
            self.ws = torch.empty(nbytes, dtype=torch.uint8, device=dev)
            w1b = I * H * 2 + M * H * 2 + M * I * 2
            w2b = H * I * 2 + M * I * 2 + M * H * 2
            self.ops = [
                ("column_gemm_decode", 2.0 * M * I * H, w1b,
                 lambda: tl.tp_linear_column(self.X1, self.W1, self.Y1, P)),
                ("row_gemm_fused_fold", 2.0 * M * H * I, w2b,
                 lambda: tl.tp_linear_row(self.X2, self.W2, self.Y2, P, tl.TP_ROW_FUSED, self.ws)),
            ]
            self.name = "decode M=16, hidden 8192, intermediate 28672, P=8; column fc1 + " \
                        "row fc2 with the fold fused into the GEMM epilogue"
            self.shape = dict(M=M, hidden=H, intermediate=I, P=P)
        elif wid == 6:
            M, H, I = 4096, 4096, 14336
            self.X1, self.W1 = nb(0, 0, (M, H), sx), nb(0, 1, (2 * I, H), sw)
            self.b1 = nb(0, 2, (2 * I,), sw)
            self.W2, self.b2 = nb(1, 1, (H, I), sw), nb(1, 2, (H,), sw)
            self.H = torch.empty((M, I), dtype=bf, device=dev)
            self.Y2 = torch.empty((M, H), dtype=bf, device=dev)
            self.parts = torch.empty((P, M, H), dtype=torch.float32, device=dev)
            # The row layer as its two explicit stages: fp32 partials, then
            # the fold with the Partial bias (TP_ROW_FUSED would fold inside
            # the GEMM at this shape; the step keeps the fold kernel with the
            # bias measured).
            self.ops = [
                ("column_gemm_swiglu_bias", 2.0 * M * 2 * I * H, None,
                 lambda: tl.tp_linear_column_ex(self.X1, self.W1, self.H, P, bias=self.b1,
                                                act=tl.TP_ACT_SWIGLU)),
                ("row_gemm", 2.0 * M * H * I, None,
                 lambda: tl.tp_linear_row(self.H, self.W2, self.parts, P, tl.TP_ROW_PARTIAL)),
                ("shard_fold_bias", 0.0, P * M * H * 4 + M * H * 2,
                 lambda: tl.tp_shard_reduce_ex(self.parts, self.Y2, P, bias=self.b2)),
            ]
            self.name = ("Llama-8B MLP TP layer: M=4096, hidden 4096, intermediate 14336, P=8; "
                         "fc1 gate+up column 4096->2x14336 with Shard(0) bias and silu(gate)*up "
                         "fused, fc2 row 14336->4096 on the gated output: fp32 shard partials, "
                         "then the shard fold with the Partial bias added once")
            self.shape = dict(M=M, hidden=H, intermediate=I, P=P)
        elif wid == 8:
            T, V, D = 4096, 128256, 4096
            Ds = D // P
            g = torch.Generator(device=dev)
            g.manual_seed(synth.seed_for(8, 0, 0))
            # A new batch of token ids every step (16 batches in turn): the
            # rows they gather (~400 MB over the 16) do not stay in the
            # 256 MB last-level cache between steps, as one fixed batch would.
            self.id_sets = [torch.randint(0, V, (T,), generator=g, device=dev, dtype=torch.int64)
                            for _ in range(16)]
            self.ids = self.id_sets[0]       # the batch of the latest lookup
            self._next_ids = 0
            self.E = [nb(0, 1 + i, (V, Ds), sx) for i in range(P)]
            self.Y1 = torch.empty((T, D), dtype=bf, device=dev)

            def lookup():
                self.ids = self.id_sets[self._next_ids]
                self._next_ids = (self._next_ids + 1) % len(self.id_sets)
                tl.tp_embedding(self.ids, self.Y1, P, e_shards=self.E)

            self.ops = [("embedding_lookup_allgather", 0.0, T * D * 2 * 2 + T * 8, lookup)]
            self.name = ("Llama-8B token embedding, EmbeddingWithReplicateOutput: vocab 128256, "
                         "hidden 4096 Shard(1) over P=8 shard tables, T=4096 token ids, "
                         "all-gathered output")
            self.shape = dict(T=T, vocab=V, hidden=D, P=P)
        else:
            M, K, N, N3 = 16384, 28672, 8192, 28672
            self.X1, self.W1 = nb(0, 0, (M, K), sx), nb(0, 1, (N, K), sw)
            self.W3 = nb(1, 1, (N3, N), sw)
            self.parts = torch.empty((P, M, N), dtype=torch.float32, device=dev)
            self.Y = torch.empty((M, N), dtype=bf, device=dev)   # slices = row blocks
            self.Y3 = torch.empty((M, N3), dtype=bf, device=dev)
            if wid == 5:
                self.ops = [
                    ("row_gemm", 2.0 * M * N * K, None,
                     lambda: tl.tp_linear_row(self.X1, self.W1, self.parts, P, tl.TP_ROW_PARTIAL)),
                    ("reduce_scatter_fold", 0.0, P * M * N * 4 + M * N * 2,
                     lambda: tl.tp_shard_reduce(self.parts, self.Y, P, scatter=1)),
                    ("column_gemm_allgathered", 2.0 * M * N3 * N, None,
                     lambda: tl.tp_linear_column(self.Y, self.W3, self.Y3, P)),
                ]
                self.name = "sequence-parallel: M=16384, K=28672 split P=8, N=8192; row GEMM, " \
                            "reduce-scatter over tokens, all-gather view -> column 8192->28672"
            else:
                # Token slices in P separate allocations, as P ranks would hold them.
                self.slices = [torch.empty((M // P, N), dtype=bf, device=dev) for _ in range(P)]
                self.ops = [
                    ("row_gemm", 2.0 * M * N * K, None,
                     lambda: tl.tp_linear_row(self.X1, self.W1, self.parts, P, tl.TP_ROW_PARTIAL)),
                    ("reduce_scatter_fold_to_slices", 0.0, P * M * N * 4 + M * N * 2,
                     lambda: tl.tp_shard_reduce_ex(self.parts, None, P, scatter=1,
                                                   y_slices=self.slices)),
                    ("column_gemm_gathered_slices", 2.0 * M * N3 * N, None,
                     lambda: tl.tp_linear_column_ex(None, self.W3, self.Y3, P,
                                                    x_slices=self.slices)),
                ]
                self.name = "sequence-parallel, slices in separate allocations: M=16384, " \
                            "K=28672 split P=8, N=8192; row GEMM, reduce-scatter into 8 slice " \
                            "allocations, column 8192->28672 reading the slices in place"
            self.shape = dict(M=M, K=K, N=N, N_next=N3, P=P)
        self.flops = sum(op[1] for op in self.ops)
        self.single = self._single_shard_ops(P, torch, tl)

    def _single_shard_ops(self, P, torch, tl):
        """Each GEMM's shards launched alone, one at a time, at their real
        shape (one GPU's share of the layer): (name, flop, bytes, fns) with
        one launch function per shard.  The timer takes the shards in turn,
        so a shard's operands (58.7 MB for a decode shard) are not still in
        the 256 MB last-level cache from the launch before.  Timed outside
        the step."""
        dev, bf = "cuda:0", torch.bfloat16
        ops = []
        def col(name, X, W):
            Ns = W.shape[0] // P
            Y = torch.empty((X.shape[0], Ns), dtype=bf, device=dev)
            fl = 2.0 * X.shape[0] * Ns * X.shape[1]
            nb = (Ns * X.shape[1] + X.numel() + Y.numel()) * 2
            fns = [lambda Wi=W[i * Ns:(i + 1) * Ns]: tl.tp_linear_column(X, Wi, Y, 1)
                   for i in range(P)]
            ops.append((name, fl, nb, fns))
        def row(name, X, W, fused):
            Ks = X.shape[1] // P
            M, N = X.shape[0], W.shape[0]
            sl = [(X[:, i * Ks:(i + 1) * Ks], W[:, i * Ks:(i + 1) * Ks]) for i in range(P)]
            fl = 2.0 * M * N * Ks
            if fused:
                Y = torch.empty((M, N), dtype=bf, device=dev)
                ws = torch.empty(tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, M, N, 1),
                                 dtype=torch.uint8, device=dev)
                nb = (N * Ks + M * Ks + Y.numel()) * 2
                fns = [lambda a=a, b=b: tl.tp_linear_row(a, b, Y, 1, tl.TP_ROW_FUSED, ws)
                       for a, b in sl]
            else:
                part = torch.empty((1, M, N), dtype=torch.float32, device=dev)
                nb = (N * Ks + M * Ks) * 2 + part.numel() * 4
                fns = [lambda a=a, b=b: tl.tp_linear_row(a, b, part, 1, tl.TP_ROW_PARTIAL)
                       for a, b in sl]
            ops.append((name, fl, nb, fns))
        if self.wid in (2, 3):
            col("column_gemm_one_shard", self.X1, self.W1)
            row("row_gemm_one_shard", self.X2, self.W2, False)
            # the whole row layer (all P shards) through TP_ROW_FUSED, launched
            # back to back: the library folds inside the GEMM where that is
            # faster (both layers here: shard K 1792 and 1024), else runs
            # partials + fold
            M, N = self.X2.shape[0], self.W2.shape[0]
            Yf = torch.empty((M, N), dtype=bf, device=dev)
            wsf = torch.empty(tl.tp_row_workspace_bytes(tl.TP_ROW_FUSED, M, N, P),
                              dtype=torch.uint8, device=dev)
            ops.append(("row_layer_tp_row_fused_all_shards", 2.0 * M * N * self.X2.shape[1], None,
                        [lambda: tl.tp_linear_row(self.X2, self.W2, Yf, P, tl.TP_ROW_FUSED, wsf)]))
        elif self.wid == 4:
            col("column_gemm_decode_one_shard", self.X1, self.W1)
            row("row_gemm_decode_one_shard", self.X2, self.W2, True)
        elif self.wid == 6:
            X, W, b = self.X1, self.W1, self.b1
            Ns = W.shape[0] // P
            Hs = torch.empty((X.shape[0], Ns // 2), dtype=bf, device=dev)
            fl = 2.0 * X.shape[0] * Ns * X.shape[1]
            nb = (Ns * X.shape[1] + X.numel() + Hs.numel()) * 2
            fns = [lambda Wi=W[i * Ns:(i + 1) * Ns], bi=b[i * Ns:(i + 1) * Ns]:
                   tl.tp_linear_column_ex(X, Wi, Hs, 1, bias=bi, act=tl.TP_ACT_SWIGLU)
                   for i in range(P)]
            ops.append(("column_gemm_swiglu_bias_one_shard", fl, nb, fns))
            row("row_gemm_one_shard", self.H, self.W2, False)
        elif self.wid in (5, 7):
            row("row_gemm_one_shard", self.X1, self.W1, False)
            col("column_gemm_allgathered_one_shard", self.Y, self.W3)
        return ops


def traffic_bytes(wid, op):
    """HBM-side bytes per launch of `op` measured by the rocprofv3 counter
    passes summarised in profiles/traffic.json, or None when there is no
    record or the kernel's source has changed since it was taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", "traffic.json")
    try:
        rec = json.load(open(path))["ops"][str(wid)][op]
    except (OSError, KeyError, ValueError):
        return None
    k = rec["kernel"]
    files = {"rowfold": "gemm_rowfold.hip", "tile": "gemm_tile.hip", "skinny": "gemm_skinny.hip",
             "fold": "shard_fold.hip", "embedding": "embedding.hip", "generic": "gemm_generic.hip"}
    srcs = next((f for key, f in files.items() if key in k), None)
    if srcs is None:
        return None
    h = hashlib.sha256()
    for f in (srcs, "kernels.h"):
        h.update(open(os.path.join(ROOT, "tensor_linear_amd", "csrc", f), "rb").read())
    return rec["bytes"] if h.hexdigest()[:16] == rec["source_sha256_16"] else None


def cpu_baseline(wl, rows, np, oracle, torch):
    """Time the oracle on the first `rows` token rows of the workload's GEMMs
    (all output columns), plus the fp32 fold over the same rows; for the
    embedding, the oracle's lookup of the first `rows` tokens.  Every oracle
    input is a workload input (or the oracle's own result of an earlier
    stage), never a result of the library."""
    def host64(t):
        return oracle.widen_bf16(t.detach().cpu().view(torch.int16).numpy().view(np.uint16))
    P = wl.P
    flops, secs, parity = 0.0, 0.0, {}
    fold_s, fold_b = 0.0, 0
    emb_b = 0
    h_oracle = None   # the oracle's own gated output, the input of workload 6's row GEMM
    for name, fl, nbytes, _ in wl.ops:
        if name in ("column_gemm", "column_gemm_decode", "column_gemm_swiglu_bias"):
            X, W = wl.X1, wl.W1
            r = min(rows, X.shape[0])
            X64, Wio = host64(X[:r]), np.ascontiguousarray(host64(W).T)
            t0 = time.perf_counter()
            if name == "column_gemm_swiglu_bias":
                Y = oracle.column_parallel_swiglu(X64, Wio, host64(wl.b1), P)
            else:
                Y = oracle.column_parallel_linear(X64, Wio, P)
            secs += time.perf_counter() - t0
            flops += fl * r / X.shape[0]
            out = wl.H if name == "column_gemm_swiglu_bias" else wl.Y1
            got = host64(out[:r])
            if name == "column_gemm_swiglu_bias":
                h_oracle = oracle.widen_bf16(oracle.round_bf16(Y.astype(np.float32)))
            parity[name] = dict(rows=r, rel_l2=oracle.rel_l2(got, Y),
                                max_abs=oracle.max_abs(got, Y))
        elif name in ("row_gemm", "row_gemm_fused_fold"):
            X, W = (wl.X1, wl.W1) if wl.wid in (5, 7) else (getattr(wl, "X2", None), wl.W2)
            Mrows = wl.shape["M"]
            r = min(rows, Mrows)
            X64 = h_oracle[:r] if wl.wid == 6 else host64(X[:r])
            Wio = np.ascontiguousarray(host64(W).T)
            t0 = time.perf_counter()
            parts = oracle.row_partials(X64, Wio, P)
            Y = oracle.fold_f64(parts)
            if wl.wid == 6:
                Y = Y + host64(wl.b2)[None, :]
            secs += time.perf_counter() - t0
            flops += fl * r / Mrows
            # the fp32 fold (and one rounding) of the oracle's own partials
            p32 = np.stack([p.astype(np.float32) for p in parts])
            t0 = time.perf_counter()
            oracle.round_bf16(oracle.fold_f32(p32))
            fold_s = time.perf_counter() - t0
            fold_b = p32.nbytes + p32[0].size * 2
            if wl.wid == 7:
                got_t = torch.cat(wl.slices)[:r]
            else:
                got_t = getattr(wl, {5: "Y"}.get(wl.wid, "Y2"))[:r]
            got = host64(got_t)
            parity[name] = dict(rows=r, rel_l2=oracle.rel_l2(got, Y),
                                max_abs=oracle.max_abs(got, Y))
        elif name == "embedding_lookup_allgather":
            r = min(rows, wl.ids.shape[0])
            ids = wl.ids[:r].cpu().numpy()
            E = np.concatenate([t.detach().cpu().view(torch.int16).numpy().view(np.uint16)
                                for t in wl.E], axis=1)
            t0 = time.perf_counter()
            Y = oracle.embedding_parallel(ids, E, P)
            secs += time.perf_counter() - t0
            emb_b += nbytes * r / wl.ids.shape[0]
            got = wl.Y1[:r].cpu().view(torch.int16).numpy().view(np.uint16)
            parity[name] = dict(rows=r, bitwise_equal=bool(np.array_equal(got, Y)))
    cpu_model = ""
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                cpu_model = line.split(":", 1)[1].strip()
                break
    except OSError:
        pass
    M = wl.shape.get("M", wl.shape.get("T"))
    if emb_b:
        value, unit = emb_b / secs / 1e9 if secs > 0 else None, "GB/s"
        what = f"lookup of the first {rows} token ids (all shards, all features)"
    else:
        value, unit = flops / secs / 1e12 if secs > 0 else None, "TFLOP/s"
        what = (f"first {rows} token rows of each GEMM (all output columns, all K), fp64 triple "
                f"loop with explicit shard split/concat/sum; {flops / 1e9:.1f} GFLOP")
    return dict(value=value, unit=unit,
                cores=oracle.num_threads(), kind="oracle",
                sample=f"{what} in {secs:.1f} s; linear in the row count, so the full workload "
                       f"takes about {secs * M / min(rows, M):.2f} s",
                fold_gbps=fold_b / fold_s / 1e9 if fold_s > 0 else None,
                cpu_model=cpu_model, os_cpu_count=os.cpu_count(),
                affinity=len(os.sched_getaffinity(0))), parity


def shader_clock(wl, op_stats, steps, step_ms, torch):
    """Shader clock (GHz) with the GPU idle, while each GEMM of the step runs
    back to back, and over a replay of the timed steps: a probe kernel
    (libtplclock.so, one wave per block) on a second stream counts s_memtime
    ticks against the 100 MHz real-time counter over a window of a few ms
    (the clock swings under load, so short windows mislead).  Outside the
    timed step; None when the probe library is not built."""
    import ctypes
    path = os.path.join(ROOT, "tensor_linear_amd", "libtplclock.so")
    if not os.path.exists(path):
        return None
    lib = ctypes.CDLL(path)
    lib.tp_clock_probe.argtypes = [ctypes.c_void_p, ctypes.c_int, ctypes.c_uint, ctypes.c_uint,
                                   ctypes.c_void_p]
    lib.tp_clock_probe.restype = ctypes.c_int
    nb, delay_us = 16, 50
    buf = torch.zeros(2 * nb, dtype=torch.int64, device="cuda:0")
    side = torch.cuda.Stream()

    def probe(fn, reps, window_us):
        torch.cuda.synchronize()
        rc = lib.tp_clock_probe(ctypes.c_void_p(buf.data_ptr()), nb, delay_us * 100,
                                int(window_us * 100), ctypes.c_void_p(side.cuda_stream))
        if rc != 0:
            raise RuntimeError(f"tp_clock_probe failed: hip error {rc}")
        for _ in range(reps):
            fn()
        torch.cuda.synchronize()
        o = buf.cpu().tolist()
        ghz = [o[2 * b] / (o[2 * b + 1] / 100e6) / 1e9 for b in range(nb)]
        return sum(ghz) / nb

    def step():
        for op in wl.ops:
            op[3]()

    out = {"idle": probe(lambda: None, 0, 500)}
    for name, fl, _, fn in wl.ops:
        if not fl:
            continue
        window = 2500
        out[name] = probe(fn, int((delay_us + window + 300) / op_stats[name]["avg_us"]) + 2, window)
    out["step_replay"] = probe(step, steps, max(1000.0, 0.8 * steps * step_ms * 1e3 - delay_us))
    return out


def platform_reference(wl, steps, torch):
    """The platform's own kernels on the same inputs, timed the way the step
    is (context, not part of the step).  GEMM workloads: the platform GEMM
    (torch.nn.functional.linear, hipBLASLt) on each column GEMM's dense
    equivalent -- X [M, K] times all N rows of W, the same flops and the same
    output -- and on the row GEMM's full-K product (the same flops, one bf16
    output instead of P fp32 partials); for decode also the rate of the bytes
    it must stream (W + X + Y).  Embedding: F.embedding of the same
    batches of ids over the P shard tables concatenated into one [V, D] table
    (the same bytes moved as the library's lookup), and the per-shard gather
    followed by torch.cat (what the same lookup costs written with torch ops
    on the shard tables); both captured with one new batch per launch in a
    HIP graph and the replay timed, as the embedding step is."""
    import torch.nn.functional as F
    out = {}

    def timed(fn, reps):
        for _ in range(3):
            fn()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        for _ in range(reps):
            fn()
        e1.record()
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) / reps * 1e3   # us

    if wl.wid in (2, 3, 4, 5, 6, 7):
        pairs = []
        if wl.wid in (2, 3):
            pairs = [("column_gemm", wl.X1, wl.W1), ("row_gemm_full_k", wl.X2, wl.W2)]
        elif wl.wid == 4:
            pairs = [("column_gemm_decode", wl.X1, wl.W1), ("row_gemm_full_k", wl.X2, wl.W2)]
        elif wl.wid in (5, 7):
            pairs = [("row_gemm_full_k", wl.X1, wl.W1), ("column_gemm", wl.Y, wl.W3)]
        elif wl.wid == 6:
            pairs = [("column_gemm_gate_up", wl.X1, wl.W1), ("row_gemm_full_k", wl.H, wl.W2)]
        for name, X, W in pairs:
            fl = 2.0 * X.shape[0] * X.shape[1] * W.shape[0]
            us = timed(lambda X=X, W=W: F.linear(X, W), max(3, min(20, int(2e13 / fl))))
            out[name] = dict(avg_us=us, tflops=fl / us / 1e6,
                             frac_bf16_peak=fl / us / 1e6 / PEAK_BF16_TFLOPS,
                             kernel="torch.nn.functional.linear (platform GEMM)")
            if wl.wid == 4:   # decode: bound by streaming W
                nbytes = (W.numel() + X.numel() + X.shape[0] * W.shape[0]) * 2
                out[name].update(algorithmic_bytes=nbytes, gbps=nbytes / us / 1e3,
                                 frac_hbm_peak=nbytes / us / 1e3 / PEAK_HBM_GBPS)
    elif wl.wid == 8:
        T, D = wl.ids.shape[0], wl.Y1.shape[1]
        nbytes = T * D * 2 * 2 + T * 8
        full = torch.cat(wl.E, dim=1)          # [V, D]: the shard tables side by side
        for name, fn in (
                ("embedding_one_table", lambda ids: F.embedding(ids, full)),
                ("embedding_shard_tables_cat",
                 lambda ids: torch.cat([F.embedding(ids, e) for e in wl.E], dim=1))):
            fn(wl.id_sets[0])
            torch.cuda.synchronize()
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn(wl.id_sets[0])
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for s in range(steps):
                    fn(wl.id_sets[s % len(wl.id_sets)])
            g.replay()
            torch.cuda.synchronize()
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            g.replay()
            e1.record()
            torch.cuda.synchronize()
            us = e0.elapsed_time(e1) / steps * 1e3
            out[name] = dict(avg_us=us, gbps=nbytes / us / 1e3, frac_hbm_peak=nbytes / us / 1e3 / PEAK_HBM_GBPS)
            del g
        del full
    return out


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU: all P shards are resident on one MI355X; "
              f"--gpus {args.gpus} is not supported", file=sys.stderr)
        sys.exit(2)
    import numpy as np
    import torch
    import synth
    import tensor_linear_amd as tl

    if args.copy_calibration:
        n = args.copy_calibration << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        for _ in range(3):
            dst.copy_(src)
        torch.cuda.synchronize()
        del src, dst

    wl = Workload(args.workload, torch, tl, synth)
    torch.cuda.synchronize()
    for _ in range(args.warmup):
        for op in wl.ops:
            op[3]()
    torch.cuda.synchronize()

    # HIP events on the launch stream.  With several ops per step an event
    # follows every op.  A one-op step (the ~16 us embedding kernel) is
    # shorter than the host's cost of one call from Python, so its K timed
    # launches are captured in a HIP graph (each with its own batch of ids)
    # and the replay is timed with one event pair: the GPU time of K steps,
    # not the host's launch rate.
    nops = len(wl.ops)
    per_op = nops > 1
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(nops + 1)]
           for _ in range(args.steps if per_op else 1)]
    graph = None
    if not per_op:
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            wl.ops[0][3]()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(graph):
            for s in range(args.steps):
                wl.ops[0][3]()
        graph.replay()                  # one untimed replay
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    if not per_op:
        evs[0][0].record()
        graph.replay()
        evs[0][1].record()
    for s in range(args.steps if per_op else 0):
        evs[s][0].record()
        for i, op in enumerate(wl.ops):
            op[3]()
            evs[s][i + 1].record()
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_step = wall / args.steps * 1e3

    op_stats = {}
    for i, (name, fl, nbytes, _) in enumerate(wl.ops):
        if per_op:
            ts = sorted(evs[s][i].elapsed_time(evs[s][i + 1]) for s in range(args.steps))
        else:
            ts = [evs[0][0].elapsed_time(evs[0][1]) / args.steps] * args.steps
        avg = sum(ts) / len(ts)
        st = dict(avg_us=avg * 1e3, min_us=ts[0] * 1e3, median_us=ts[len(ts) // 2] * 1e3)
        if fl:
            st["tflops"] = fl / (avg * 1e-3) / 1e12
            st["frac_bf16_peak"] = st["tflops"] / PEAK_BF16_TFLOPS
        if nbytes:
            st["algorithmic_bytes"] = nbytes
            st["gbps"] = nbytes / (avg * 1e-3) / 1e9
            st["frac_hbm_peak"] = st["gbps"] / PEAK_HBM_GBPS
        op_stats[name] = st

    # Context, outside the timed step: each GEMM's shards alone at their real
    # shape, in turn, and a plain device copy of 1 GiB.
    # The launches are captured in a HIP graph and the replay is timed: a
    # decode shard runs for ~10 us, less than one call from Python costs the
    # host, so eager launches would time the host.
    single = {}
    for name, fl, nb, fns in wl.single:
        reps = max(10, len(fns))
        seq = [fns[r % len(fns)] for r in range(reps)]
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for f in seq[:3]:
                f()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        sgraph = torch.cuda.CUDAGraph()
        with torch.cuda.graph(sgraph):
            for f in seq:
                f()
        sgraph.replay()                 # one untimed replay
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        sgraph.replay()
        e1.record()
        torch.cuda.synchronize()
        us = e0.elapsed_time(e1) / reps * 1e3
        del sgraph
        single[name] = dict(avg_us=us, tflops=fl / us / 1e6,
                            frac_bf16_peak=fl / us / 1e6 / PEAK_BF16_TFLOPS)
        if nb:
            single[name].update(gbps=nb / us / 1e3, frac_hbm_peak=nb / us / 1e3 / PEAK_HBM_GBPS)
    src = torch.empty(1 << 30, dtype=torch.uint8, device="cuda:0").fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(5):
        dst.copy_(src)
    e1.record()
    torch.cuda.synchronize()
    copy_gbps = 2 * (1 << 30) * 5 / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del src, dst

    clocks = shader_clock(wl, op_stats, args.steps, ms_step, torch)
    platform = platform_reference(wl, args.steps, torch) if args.platform_reference else {}

    # dominant kernel: the op with the most time
    dom = max(op_stats, key=lambda k: op_stats[k]["avg_us"])
    d = op_stats[dom]
    if "tflops" in d and wl.wid != 4:
        roof = dict(kernel=dom, bound="mfma", achieved=d["tflops"], peak=PEAK_BF16_TFLOPS,
                    unit="TFLOP/s", frac=d["tflops"] / PEAK_BF16_TFLOPS,
                    traffic=traffic_bytes(args.workload, dom),
                    avg_launch_us=d["avg_us"])
    else:
        roof = dict(kernel=dom, bound="hbm", achieved=d["gbps"], peak=PEAK_HBM_GBPS,
                    unit="GB/s", frac=d["gbps"] / PEAK_HBM_GBPS,
                    traffic=traffic_bytes(args.workload, dom),
                    avg_launch_us=d["avg_us"])

    if wl.flops:
        value, unit = wl.flops / (ms_step * 1e-3) / 1e12, "TFLOP/s"
    else:   # a pure data-movement workload (the embedding): bytes per second
        value = sum(op[2] for op in wl.ops) / (ms_step * 1e-3) / 1e9
        unit = "GB/s"
    out = {
        "metric": METRIC,
        "value": value,
        "unit": unit,
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic: X ~ N(0,1), W ~ N(0,0.02^2), bf16, drawn on the GPU from fixed seeds",
        "config": dict(workload=wl.name, **wl.shape),
        "roofline": roof,
        "ops": op_stats,
        "context": {"one_shard": single,
                    "device_copy_gbps": copy_gbps,
                    "shader_clock_ghz": clocks,
                    "note": "one_shard: each GEMM's shards launched alone at their real shape "
                            "(one GPU's share), one after another (so a shard is not still "
                            "cached from the launch before), captured in a HIP graph and the replay timed, "
                            "and for the prefill workloads the whole row layer "
                            "through TP_ROW_FUSED back to back (the fold inside the GEMM, bitwise equal to "
                            "partials + fold); device_copy_gbps: read+write bytes of a 1 GiB "
                            "device-to-device copy per second; shader_clock_ghz: the shader "
                            "clock idle, while each GEMM of the step runs back to back (2.5 ms "
                            "window) and over a replay of the timed steps, from a probe kernel "
                            "on a second stream; bf16 peak assumes "
                            f"{PEAK_CLOCK_GHZ} GHz; none of these is part of the step"},
    }
    if platform:
        out["context"]["platform_reference"] = platform
    if graph is not None:
        out["context"]["timing"] = (f"the {args.steps} timed launches captured in one HIP graph "
                                    "(a new batch of ids each) and its replay timed with one "
                                    "event pair")
    if clocks and roof["bound"] == "mfma" and dom in clocks:
        c = clocks[dom]
        peak_c = PEAK_BF16_TFLOPS * c / PEAK_CLOCK_GHZ
        out["context"]["roofline_at_measured_clock"] = dict(
            kernel=dom, clock_ghz=c, peak=peak_c, unit="TFLOP/s", frac=roof["achieved"] / peak_c)
    if not args.no_cpu_baseline:
        import oracle
        cb, parity = cpu_baseline(wl, args.cpu_rows, np, oracle, torch)
        out["cpu_baseline"] = cb
        out["parity_sample"] = parity
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
