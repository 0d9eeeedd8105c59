"""Helpers shared by the GPU tests: moving seeded inputs to the device and
results back.  No arithmetic of the method lives here."""
import contextlib
import os

import numpy as np
import torch

import oracle
import tensor_linear_amd as tl

DEV = "cuda:0"


def bf16_dev(bits: np.ndarray) -> torch.Tensor:
    """uint16 bf16 bit patterns -> bfloat16 tensor on the GPU."""
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16)
    return t.to(DEV)


def f32_dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(DEV)


def to_f64(t: torch.Tensor) -> np.ndarray:
    """Device result -> fp64 numpy, exactly."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.widen_bf16(t.view(torch.int16).numpy().view(np.uint16))
    return t.numpy().astype(np.float64)


def bits(t: torch.Tensor) -> np.ndarray:
    """Raw bit patterns of a device result (uint16 for bf16, uint32 for fp32)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy().view(np.uint32)


def expected_bits(ref64: np.ndarray, dtype) -> np.ndarray:
    """Bit patterns of an exactly known result rounded once to the output
    type (fp64 -> fp32 is exact for the integer-valued cases used)."""
    f = np.asarray(ref64, dtype=np.float32)
    if dtype == torch.bfloat16:
        return oracle.round_bf16(f)
    return f.view(np.uint32)


def workspace(mode, M, N, P, zero=True) -> torch.Tensor:
    nbytes = tl.tp_row_workspace_bytes(mode, M, N, P)
    ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=DEV)
    if zero:
        tl.tp_workspace_zero(ws)
    return ws


def bf16_tol(K: int, sx: float = 1.0, sw: float = 0.02) -> float:
    """Max-abs bar for bf16 inputs with fp32 accumulation: 2e-2 sqrt(K) sx sw."""
    return 2e-2 * np.sqrt(K) * sx * sw


# The two choices of the fused row modes: the library's own (the fold inside
# the GEMM only where that measured faster) and every shape a fused kernel
# takes (TPLINEAR_ROW_FOLD=gemm).  Both give the bits of TP_ROW_SUM.
FOLD_POLICIES = (None, "gemm")


@contextlib.contextmanager
def row_fold(policy):
    """Run the calls inside with TPLINEAR_ROW_FOLD = policy (None: unset)."""
    old = os.environ.get("TPLINEAR_ROW_FOLD")
    if policy is None:
        os.environ.pop("TPLINEAR_ROW_FOLD", None)
    else:
        os.environ["TPLINEAR_ROW_FOLD"] = policy
    try:
        yield
    finally:
        if old is None:
            os.environ.pop("TPLINEAR_ROW_FOLD", None)
        else:
            os.environ["TPLINEAR_ROW_FOLD"] = old
