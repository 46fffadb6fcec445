"""Shared helpers for the GPU tests (device transfer, tolerances, canaries)."""
import numpy as np
import torch

# Float-output tolerances (normwise: max|y - y_ref| / max|y_ref| against the
# unrounded fp64 oracle): fp32-activation paths 1e-5, bf16-activation paths
# 2e-3 (bf16 output rounding alone is up to 2^-9 relative per element).
TOL_F32 = 1e-5
TOL_BF16 = 2e-3


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def dev_bf16(bits: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint16)).cuda().view(torch.bfloat16)


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    if t.dtype == torch.bfloat16:
        return t.view(torch.uint16).cpu().numpy()
    return t.cpu().numpy()


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (np.asarray(bits, np.uint16).astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def guarded(n: int, dtype, guard: int = 64):
    """An output buffer with canary bands on both sides; returns (full, view)."""
    full = torch.empty(n + 2 * guard, dtype=dtype, device="cuda")
    full.view(torch.uint8).fill_(0x5A)
    return full, full[guard:guard + n]


def canaries_intact(full: torch.Tensor, n: int, guard: int = 64) -> bool:
    raw = full.view(torch.uint8).cpu().numpy()
    isz = full.dtype.itemsize
    head = raw[:guard * isz]
    tail = raw[(guard + n) * isz:]
    return bool(np.all(head == 0x5A) and np.all(tail == 0x5A))
