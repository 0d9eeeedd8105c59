"""Seeded synthetic inputs for the tensor-parallel Linear workloads.

This module draws random numbers and picks sample rows; it holds none of the
method's arithmetic (no products, sums, splits or rounding of results).  It
is the one piece both the HIP path's tests/bench and the CPU oracle use.

Inputs follow the workload recipe: X ~ N(0, 1), W ~ N(0, 0.02^2), drawn as
fp32 with numpy's PCG64 generator and converted to bf16 by torch's CPU cast.
Weights are produced in the [out, in] = [N, K] storage the library takes.
Seed of tensor t (0 = X, 1 = W) of GEMM g in workload c: 1000*c + 10*g + t.
"""
import numpy as np

SIGMA_X = 1.0
SIGMA_W = 0.02


def seed_for(cfg: int, gemm: int, tensor: int) -> int:
    return 1000 * cfg + 10 * gemm + tensor


def normal_f32(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(size=shape, dtype=np.float32)
    if sigma != 1.0:
        a *= np.float32(sigma)
    return a


def to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns using torch's CPU cast (a library routine)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def normal_bf16(seed: int, shape, sigma: float = 1.0) -> np.ndarray:
    """bf16 bit patterns (uint16) of N(0, sigma^2) samples."""
    return to_bf16_bits(normal_f32(seed, shape, sigma))


def small_ints(seed: int, shape, lo: int = -2, hi: int = 2) -> np.ndarray:
    """Integers in [lo, hi] as fp32 (exact in fp32 and in bf16)."""
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=shape).astype(np.float32)


def sample_rows(M: int, seed: int, block: int = 256) -> np.ndarray:
    """Row 0, one seeded row from every `block` rows, and row M-1 (sorted,
    unique).  Used where a full-size reference product would take too long:
    each output row depends only on its own input row."""
    rng = np.random.default_rng(seed)
    rows = {0, M - 1}
    for b0 in range(0, M, block):
        rows.add(int(rng.integers(b0, min(b0 + block, M))))
    return np.array(sorted(rows), dtype=np.int64)


# The workloads: (name, M, K, N, P) per GEMM; dtype bf16 unless stated.
WORKLOADS = {
    1: dict(name="worked example X 3x8, W 8x12, P=4 (fp32)",
            gemms=[("column", 3, 8, 12, 4), ("row", 3, 8, 12, 4)], dtype="f32"),
    2: dict(name="Llama-8B MLP TP shard M=4096 P=8",
            gemms=[("column", 4096, 4096, 2 * 14336, 8),      # fc1 gate+up
                   ("row", 4096, 14336, 4096, 8)], dtype="bf16"),  # fc2
    3: dict(name="Llama-70B attention TP shard M=8192 P=8",
            gemms=[("column", 8192, 8192, 10240, 8),          # fused QKV
                   ("row", 8192, 8192, 8192, 8)], dtype="bf16"),   # O
    4: dict(name="decode M=16 hidden 8192 intermediate 28672 P=8",
            gemms=[("column", 16, 8192, 28672, 8),
                   ("row_fused", 16, 28672, 8192, 8)], dtype="bf16"),
    5: dict(name="sequence-parallel M=16384 K=28672 N=8192 P=8",
            gemms=[("row_scatter", 16384, 28672, 8192, 8),
                   ("column", 16384, 8192, 28672, 8)], dtype="bf16"),
}


def device_normal_bf16(seed: int, shape, sigma: float, device="cuda:0"):
    """N(0, sigma^2) bf16 tensor drawn on the GPU with torch's seeded
    generator (used where only throughput is measured and the inputs are too
    large to draw on the host quickly)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    t = torch.randn(shape, generator=g, device=device, dtype=torch.float32)
    if sigma != 1.0:
        t.mul_(sigma)
    return t.to(torch.bfloat16)
