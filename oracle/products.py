"""Integer and fp64 reference products (test infrastructure only).

Integer products are exact.  ``int_dot_exact`` / ``int_gemm_exact`` use an
fp64 matrix product on integer-valued operands: every product and every
partial sum is an integer of magnitude <= K * 127 * 127 < 2**53, so each
floating-point operation is exact whatever order the library sums in.  The
bound is asserted.  ``int_dot_bruteforce`` is the same sum with Python ints.

Float references are fp64 "dequantize, then multiply" computed from the
oracle's own codes and scales ([VG] 'Symmetric quantization', Fig. 19:
x_hat = x_q / s; [VG] 'BitNet', output dequantization Fig. 57: the integer
product is rescaled by the weight and activation scales).
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f32

_EXACT = float(2 ** 53)


def _check_exact(k: int, amax_a: int, amax_b: int):
    if k * amax_a * amax_b >= _EXACT:
        raise OverflowError("fp64 product would not be exact")


def int_dot_exact(wq: np.ndarray, xq: np.ndarray) -> np.ndarray:
    """acc[n] = sum_k wq[n,k] * xq[k], exact, int64."""
    wq = np.asarray(wq)
    xq = np.asarray(xq)
    k = wq.shape[-1]
    _check_exact(k, 128, 128)
    acc = wq.astype(np.float64) @ xq.astype(np.float64)
    return acc.astype(np.int64)


def int_gemm_exact(xq: np.ndarray, wq: np.ndarray) -> np.ndarray:
    """acc[m,n] = sum_k xq[m,k] * wq[n,k], exact, int64 (both operands K-contiguous)."""
    xq = np.asarray(xq)
    wq = np.asarray(wq)
    _check_exact(xq.shape[1], 128, 128)
    acc = xq.astype(np.float64) @ wq.astype(np.float64).T
    return acc.astype(np.int64)


def int_dot_bruteforce(wq, xq):
    """Same sum with Python integers, one term at a time (small inputs)."""
    out = []
    for row in np.atleast_2d(np.asarray(wq)):
        s = 0
        for a, b in zip(row.tolist(), np.asarray(xq).tolist()):
            s += int(a) * int(b)
        out.append(s)
    return np.array(out, dtype=np.int64)


def y_w8a8(acc, s_w, s_x) -> np.ndarray:
    """W8A8 output: y[n] = acc[n] / (s_w[n] * s_x) in fp64 ([VG] 'Why quantize
    activations': W8A8 runs the product on int8 weights and activations)."""
    return np.asarray(acc, np.float64) / (np.asarray(s_w, np.float64) * np.float64(np.asarray(s_x).ravel()[0]))


def y_w8a16(wq, s_w, x_bf16_bits) -> np.ndarray:
    """Weight-only int8 output: y[n] = sum_k (wq[n,k] / s_w[n]) * x[k], fp64,
    x the bf16 activation ([VG] 'Why quantize activations': weight-only
    schemes keep 16-bit activations; [OVR] section 6.2 quantizes weights
    first and keeps activations in 16 bits)."""
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    return (np.asarray(wq, np.float64) @ x) / np.asarray(s_w, np.float64)


def y_w8a16_batch(wq, s_w, x_bf16_bits) -> np.ndarray:
    """Weight-only int8 output for a small batch of M tokens (decode of
    several sequences at once; [SEP] section 3.1: at batch 1 the weights are
    read once per token, so a batch reads them once for all M tokens):
    y[t][n] = sum_k (wq[n,k] / s_w[n]) * x[t][k], fp64; x [M][K] bf16 bits,
    y [M][N]."""
    x = bf16_bits_to_f32(np.asarray(x_bf16_bits, np.uint16)).astype(np.float64)
    if x.ndim != 2:
        raise ValueError("x must be [M][K]")
    return (x @ np.asarray(wq, np.float64).T) / np.asarray(s_w, np.float64)[None, :]


def y_ternary(acc, gamma, s_x) -> np.ndarray:
    """Ternary output: y[n] = gamma * acc[n] / s_x, fp64 ([VG] 'BitNet b1.58':
    ternary weights add, skip or subtract each int8 activation; the sum is
    rescaled by the weight scale gamma and the activation scale)."""
    return np.asarray(acc, np.float64) * np.float64(gamma) / np.float64(np.asarray(s_x).ravel()[0])


def y_sign_residual(sign, alpha, rq, s_r, x_bf16_bits) -> np.ndarray:
    """Separated-quantization output: y = alpha * (sign . x) + (rq . x) / s_r,
    fp64 ([SEP] sections 1.3 and 2.3: the backbone and residual products are
    computed and their results added)."""
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    b = np.asarray(sign, np.float64) @ x
    r = np.asarray(rq, np.float64) @ x
    return np.asarray(alpha, np.float64) * b + r / np.asarray(s_r, np.float64)


def y_sign_residual_zp(sign, alpha, rq, s_r, z_r, x_bf16_bits) -> np.ndarray:
    """Output with the zero-point residual: y = alpha * (sign . x) +
    ((rq - z_r) . x) / s_r, fp64 ([SEP] sections 2.3 and 6.3; [VG]
    'Asymmetric quantization', fig. 25: subtract the zero-point, then divide
    by the scale)."""
    x = bf16_bits_to_f32(x_bf16_bits).astype(np.float64)
    b = np.asarray(sign, np.float64) @ x
    r = (np.asarray(rq, np.float64) - np.asarray(z_r, np.float64)[:, None]) @ x
    return np.asarray(alpha, np.float64) * b + r / np.asarray(s_r, np.float64)


def y_prefill(acc, s_x, s_w, x_out_bits, w_out_bits) -> np.ndarray:
    """Prefill output with the outlier path: Y = acc / (s_x[m] * s_w[n]) +
    X_out . W_out^T in fp64 ([SEP] section 2.2: outlier channels run in high
    precision, the rest in int8, and the two contributions are summed)."""
    acc = np.asarray(acc, np.float64)
    y = acc / (np.asarray(s_x, np.float64)[:, None] * np.asarray(s_w, np.float64)[None, :])
    if np.asarray(x_out_bits).size:
        xo = bf16_bits_to_f32(x_out_bits).astype(np.float64)
        wo = bf16_bits_to_f32(w_out_bits).astype(np.float64)
        y = y + xo @ wo.T
    return y


def normwise_error(y, y_ref) -> float:
    """max|y - y_ref| / max|y_ref| (the float-output tolerance measure)."""
    y = np.asarray(y, np.float64)
    y_ref = np.asarray(y_ref, np.float64)
    den = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y - y_ref)) if y_ref.size else 0.0
    return float(num / den) if den > 0 else float(num)


def relative_method_error(y_quant, w, x) -> float:
    """||y_quant - W x||_2 / ||W x||_2 against the unquantized fp64 product.

    A diagnostic of how much each format loses ([SEP] section 4.2 argues the
    residual restores what the sign backbone drops).  Reported, not graded:
    parity unpinned."""
    y_full = np.asarray(w, np.float64) @ np.asarray(x, np.float64)
    return float(np.linalg.norm(np.asarray(y_quant, np.float64) - y_full) / np.linalg.norm(y_full))
