"""Shared helpers for the GPU tests (device transfer, tolerances, canaries)."""
import numpy as np
import torch

# Float-output tolerances (normwise: max|y - y_ref| / max|y_ref| against the
# unrounded fp64 oracle): fp32-activation paths 1e-5, bf16-activation paths
# 2e-3.  A correctly rounded bf16 output carries up to half a bf16 ulp, i.e.
# up to 2^-8 relative per element (bf16 keeps 8 significant bits), so bf16
# outputs are checked by check_bf16_output below: the fp32 result against the
# tolerance, and the bf16 value as the exact RNE of that fp32 result.
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


def f32_to_bf16_rne(y32: np.ndarray) -> np.ndarray:
    """Test-side RNE narrowing used to check the kernel's own bf16 rounding."""
    u = np.ascontiguousarray(y32, np.float32).view(np.uint32).astype(np.uint64)
    return ((u + 0x7FFF + ((u >> 16) & 1)) >> 16).astype(np.uint16)


def check_bf16_output(y_bf16_bits: np.ndarray, y32: np.ndarray, y_ref: np.ndarray, tol: float = TOL_BF16):
    """bf16-output check.

    A correctly rounded bf16 value carries up to half a bf16 ulp of error
    (bf16 unit roundoff is 2^-8), so the tolerance applies to what the kernel
    computes before the output conversion: (1) its fp32 result is within `tol`
    normwise of the fp64 reference; (2) the bf16 output is exactly the RNE of
    that fp32 result; (3) elementwise, |y_bf16 - y_ref| <= half a bf16 ulp of
    y_ref + tol * max|y_ref|."""
    y_ref = np.asarray(y_ref, np.float64)
    yb = bf16_to_f64(y_bf16_bits)
    den = np.max(np.abs(y_ref))
    assert np.max(np.abs(np.asarray(y32, np.float64) - y_ref)) <= tol * den, "fp32 result outside tolerance"
    assert np.array_equal(np.asarray(y_bf16_bits, np.uint16), f32_to_bf16_rne(y32)), "bf16 output is not RNE(fp32)"
    half_ulp = np.ldexp(1.0, np.frexp(np.abs(y_ref))[1] - 9)
    assert np.all(np.abs(yb - y_ref) <= half_ulp * (1 + 1e-6) + tol * den), "bf16 output outside bound"
