"""Quantizers of the oracle (test infrastructure only).

Every step is written in the order its definition gives, in IEEE fp32 where
the definition produces an fp32 quantity (a scale, a scaled value) and in
exact arithmetic elsewhere.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f32, f32_to_bf16_bits, mean_abs_f32, mean_abs_rows_f32

Q_MAX = 127  # 2**(b-1) - 1 for b = 8 ([VG] 'Symmetric quantization', Fig. 17)


def absmax_scale(alpha: np.ndarray) -> np.ndarray:
    """s = q_max / alpha in fp32, alpha = max|x| of the group.

    [VG] 'Symmetric quantization' (absmax, Fig. 16-17): the scale is the
    multiplier q_max / alpha.  [OVR] section 3.1 step 2 writes the reciprocal
    (alpha / 127, then divides); the stored value here is the multiplier.
    An all-zero group (alpha = 0) gets s = 1 so its codes are 0 (the pages do
    not cover it).  A group so small that q_max / alpha exceeds the fp32
    range (alpha below about 3.7e-37) gets s = FLT_MAX: the quotient is
    clamped to the largest finite fp32, so every code stays finite, zeros
    stay 0 and the codes still follow round(s * x)."""
    alpha = np.asarray(alpha, dtype=np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        s = np.minimum(np.float32(Q_MAX) / alpha, np.finfo(np.float32).max)
    return np.where(alpha == np.float32(0), np.float32(1), s).astype(np.float32)


def quantize_with_scale(x: np.ndarray, s) -> np.ndarray:
    """x_q = clip(round(s * x), -q_max, q_max) with one fp32 multiply and
    round-half-to-even ([VG] 'Symmetric quantization', Fig. 17-18)."""
    x = np.asarray(x, dtype=np.float32)
    t = (x * np.asarray(s, dtype=np.float32)).astype(np.float32)
    q = np.clip(np.rint(t), -Q_MAX, Q_MAX)
    return q.astype(np.int8)


def quantize_absmax(x: np.ndarray, per_row: bool):
    """Symmetric absmax int8 quantization.

    per_row=True: one scale per row (per output channel for weights, per token
    for activations -- [OVR] section 2.3 granularity; [SEP] section 6.2 keeps a
    scale per row).  per_row=False: one scale for the whole tensor.
    Returns (codes int8, same shape as x; s fp32 [rows] or [1])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim == 1:
        x2 = x[None, :]
    else:
        x2 = x
    if per_row:
        alpha = np.max(np.abs(x2), axis=1) if x2.shape[1] else np.zeros(x2.shape[0], np.float32)
        s = absmax_scale(alpha)
        q = quantize_with_scale(x2, s[:, None])
    else:
        alpha = np.max(np.abs(x2)) if x2.size else np.float32(0)
        s = absmax_scale(np.array([alpha], dtype=np.float32))
        q = quantize_with_scale(x2, s[0])
    return q.reshape(x.shape), s.astype(np.float32)


def dequantize(q: np.ndarray, s) -> np.ndarray:
    """x_hat = x_q / s in fp64 ([VG] 'Symmetric quantization', Fig. 19)."""
    return np.asarray(q, dtype=np.float64) / np.asarray(s, dtype=np.float64)


def ternary_absmean(w: np.ndarray):
    """BitNet b1.58 absmean quantization to {-1, 0, +1} for the whole tensor.

    [VG] 'BitNet b1.58' (Fig. 60): gamma is the mean absolute weight; each
    weight is divided by gamma, rounded and clipped to [-1, 1].  gamma is the
    correctly rounded fp32 of the exact mean; W / gamma is one fp32 division;
    rounding is half-to-even.  gamma = 0 (all-zero tensor) gives all-zero codes.
    Returns (codes int8, gamma fp32)."""
    w = np.asarray(w, dtype=np.float32)
    gamma = mean_abs_f32(w) if w.size else np.float32(0)
    if gamma == 0:
        return np.zeros(w.shape, np.int8), np.float32(0)
    with np.errstate(over="ignore"):
        t = (w / gamma).astype(np.float32)
    q = np.clip(np.rint(t), -1, 1).astype(np.int8)
    return q, np.float32(gamma)


def sign_residual_split(w: np.ndarray):
    """Separated quantization of a weight matrix into a sign backbone and an
    int8 residual, per output row.

    [SEP] section 2.1: W ~ alpha * sign(W) + W_res with W_res = W - alpha*sign(W),
    and the residual is itself quantized to 8 bits with a scale of its own
    ([SEP] section 6.3).  sign maps negatives to -1 and non-negatives (incl.
    -0.0) to +1 ([VG] 'BitNet, weight quantization', Fig. 55); alpha of a row is
    its mean |W| (the least-squares optimum of ||W - alpha*sign(W)||^2) as a
    correctly rounded fp32; R = fl32(W - alpha*sign); (Rq, s_r) = per-row
    absmax int8 of R.
    Returns (sign int8 +-1, alpha fp32 [n], rq int8 [n][k], s_r fp32 [n])."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("2-D weight expected")
    sign = np.where(w >= np.float32(0), 1, -1).astype(np.int8)
    alpha = mean_abs_rows_f32(w) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    backbone = (alpha[:, None] * sign.astype(np.float32)).astype(np.float32)
    r = (w - backbone).astype(np.float32)
    rq, s_r = quantize_absmax(r, per_row=True)
    return sign, alpha, rq, s_r


Q_MIN_ASYM, Q_MAX_ASYM = -128, 127  # the int8 range the asymmetric form maps onto ([OVR] section 3 item 2)


def asym_params(lo, hi):
    """Scale and zero-point of asymmetric int8 quantization, per group.

    [VG] 'Asymmetric quantization' (figs. 22-26), in its multiplier notation:
    the float minimum beta and maximum alpha go to the ends of [q_min, q_max],
    s = (q_max - q_min) / (alpha - beta), z = round(q_min - s * beta).
    Readings: the range is widened to contain 0 (beta = min(lo, 0),
    alpha = max(hi, 0)), so that 0 is representable exactly and z lies in
    [q_min, q_max] (any range the data straddles 0 with is unchanged); an
    all-zero group (alpha = beta = 0) gets s = 1, z = q_min.  fp32 steps:
    d = fl32(alpha - beta), s = fl32(255 / d), z = rint(fl32(q_min - fl32(s * beta)))
    clipped to [q_min, q_max] (the clip is inactive up to rounding).  As for
    the symmetric scale, s is clamped to FLT_MAX when 255 / d overflows
    (d below about 7.5e-37).
    lo, hi: fp32 arrays of group minima / maxima.  Returns (s fp32, z int32)."""
    lo = np.minimum(np.asarray(lo, np.float32), np.float32(0))
    hi = np.maximum(np.asarray(hi, np.float32), np.float32(0))
    d = (hi - lo).astype(np.float32)
    with np.errstate(divide="ignore", over="ignore"):
        s = np.minimum(np.float32(Q_MAX_ASYM - Q_MIN_ASYM) / d, np.finfo(np.float32).max).astype(np.float32)
    s = np.where(d == np.float32(0), np.float32(1), s).astype(np.float32)
    t = (s * lo).astype(np.float32)
    z = np.rint((np.float32(Q_MIN_ASYM) - t).astype(np.float32))
    z = np.clip(z, Q_MIN_ASYM, Q_MAX_ASYM).astype(np.int32)
    return s, z


def quantize_with_zero_point(x: np.ndarray, s, z) -> np.ndarray:
    """x_q = clip(round(s * x + z), q_min, q_max): one fp32 multiply, one fp32
    add, round-half-to-even ([VG] 'Asymmetric quantization', fig. 24)."""
    x = np.asarray(x, dtype=np.float32)
    t = (x * np.asarray(s, dtype=np.float32)).astype(np.float32)
    u = (t + np.asarray(z, dtype=np.float32)).astype(np.float32)
    return np.clip(np.rint(u), Q_MIN_ASYM, Q_MAX_ASYM).astype(np.int8)


def quantize_asym(x: np.ndarray):
    """Asymmetric int8 quantization with one (s, z) per row of x [rows][cols].
    Returns (codes int8 [rows][cols], s fp32 [rows], z int32 [rows])."""
    x = np.asarray(x, dtype=np.float32)
    if x.ndim != 2:
        raise ValueError("2-D input expected")
    if x.shape[1]:
        lo, hi = x.min(axis=1), x.max(axis=1)
    else:
        lo = hi = np.zeros(x.shape[0], np.float32)
    s, z = asym_params(lo, hi)
    return quantize_with_zero_point(x, s[:, None], z[:, None]), s, z


def dequantize_asym(q, s, z) -> np.ndarray:
    """x_hat = (x_q - z) / s in fp64 ([VG] 'Asymmetric quantization', fig. 25)."""
    return (np.asarray(q, np.float64) - np.asarray(z, np.float64)) / np.asarray(s, np.float64)


def sign_residual_split_zp(w: np.ndarray):
    """The sign backbone of sign_residual_split with an asymmetric int8
    residual: [SEP] section 6.3 gives the residual its own min / max, scale
    and zero-point.  sign and alpha as in sign_residual_split;
    R = fl32(W - alpha * sign); (rq, s_r, z_r) = quantize_asym(R) per row.
    Returns (sign int8 +-1, alpha fp32 [n], rq int8 [n][k], s_r fp32 [n], z_r int32 [n])."""
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("2-D weight expected")
    sign = np.where(w >= np.float32(0), 1, -1).astype(np.int8)
    alpha = mean_abs_rows_f32(w) if w.shape[1] else np.zeros(w.shape[0], np.float32)
    r = (w - (alpha[:, None] * sign.astype(np.float32)).astype(np.float32)).astype(np.float32)
    rq, s_r, z_r = quantize_asym(r)
    return sign, alpha, rq, s_r, z_r


def outlier_split_quantize(x_bf16_bits: np.ndarray, idx: np.ndarray):
    """Activation outlier-channel split with per-token int8 quantization.

    [SEP] section 2.2: the few channels whose activations are tens of times
    larger are taken out and kept in high precision (here bf16, gathered
    into X_out[m][j] = X[m][idx[j]]); the remaining channels are quantized to
    int8.  The per-token absmax covers only the non-outlier channels and the
    outlier columns of Xq are 0.
    Returns (xq int8 [m][k], s_x fp32 [m], x_out bf16 bits [m][n_out])."""
    xb = np.asarray(x_bf16_bits, dtype=np.uint16)
    x = bf16_bits_to_f32(xb)
    m, k = x.shape
    idx = np.asarray(idx, dtype=np.int64)
    is_out = np.zeros(k, dtype=bool)
    is_out[idx] = True
    keep = ~is_out
    if keep.any():
        alpha = np.max(np.abs(x[:, keep]), axis=1)
    else:
        alpha = np.zeros(m, np.float32)
    s = absmax_scale(alpha)
    xq = quantize_with_scale(x, s[:, None])
    xq[:, is_out] = 0
    x_out = np.ascontiguousarray(xb[:, idx])
    return xq, s, x_out


def gather_outlier_weights(w: np.ndarray, idx: np.ndarray) -> np.ndarray:
    """W_out[n][j] = bf16(W[n][idx[j]]): the high-precision weights that the
    outlier channels multiply ([SEP] section 2.2, high-precision path).
    Returns bf16 bit patterns [n][n_out]."""
    w = np.asarray(w, dtype=np.float32)
    return f32_to_bf16_bits(np.ascontiguousarray(w[:, np.asarray(idx, dtype=np.int64)]))


def detect_outlier_channels(x_bf16_bits: np.ndarray, n_out: int) -> np.ndarray:
    """The activation channels to split out, found once from calibration
    activations ([SEP] section 2.2: a few channels are tens of times larger
    than the rest; the list is found once and cached).  The pages give no
    criterion; with a fixed budget of n_out channels the plain reading is:
    a channel's range is its max |x| over the calibration rows, and the n_out
    channels with the largest ranges are taken, equal ranges going to the
    lower channel index.
    Returns the chosen channel indices, int32, ascending."""
    x = bf16_bits_to_f32(np.asarray(x_bf16_bits, dtype=np.uint16))
    if x.ndim != 2:
        raise ValueError("2-D activations expected")
    k = x.shape[1]
    if not 0 <= n_out <= k:
        raise ValueError("n_out out of range")
    rng = np.max(np.abs(x), axis=0) if x.shape[0] else np.zeros(k, np.float32)
    order = sorted(range(k), key=lambda c: (-float(rng[c]), c))  # largest range first, then lower index
    return np.array(sorted(order[:n_out]), dtype=np.int32)
