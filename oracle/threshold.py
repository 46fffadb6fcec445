"""Thresholded separated quantization (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[SEP] section 2.1: rather than giving every weight a sign backbone, only the
weights whose magnitude is above a threshold go into the 1-bit backbone and
the rest are left to the residual.  Section 5.2: the threshold is a
percentile of |W| (the 70th or 80th; 80th is the suggested start), and the
weights above it form the backbone.  Section 5.3 (sep_linear): the backbone
is sign(W) on those weights times a scale, the residual is the 8-bit
quantization of the remaining weights, and the two products are added.
Section 3.3: residual entries near zero are set to zero under a small
threshold and the residual is stored sparse (typically 50-70% sparse); a
fast mode may skip the residual product altogether.

Readings where the pages leave the procedure open:
  * everything is per output row (the scales of [SEP] section 6.2 are per
    row);
  * a percentile is the nearest-rank one: for an integer P in 1..100 the
    P-th percentile of the K magnitudes of a row is the j-th smallest with
    j = ceil(P * K / 100), the smallest magnitude that at least P% of the
    row does not exceed;
  * backbone B = {|w| > tau}, tau = the P_b-th percentile; zero class
    Z = {|w| <= eps}, eps = the P_z-th percentile (Z is empty for P_z = 0);
    residual R = the rest, eps < |w| <= tau.  Equal magnitudes fall on the
    same side of each threshold;
  * the backbone scale alpha is the mean |w| over B (the least-squares
    scale of a sign backbone on B), correctly rounded to fp32; 0 if B is
    empty.  The sign of a backbone weight is that of w (w != 0 on B);
  * backbone weights carry no residual (sep_linear splits the weights
    between the two paths); the residual is int8 with its own per-row
    absmax scale over R: s_r = fl32(127 / max_R |w|) (1 if that max is 0 or
    R is empty), q = clip(rne(fl32(w * s_r)), -127, 127);
  * activations are per-tensor absmax int8 (the residual product is an int8
    matrix product); y = alpha * acc_b / s_x + acc_r / (s_r * s_x) with
    acc_b = sum_B sign(w) x_q and acc_r = sum_R q x_q exact integers.

Storage (this library's layout):
  class plane [N][K/4] bytes: a 2-bit field per weight, that of weight k in
      byte k/4 at bits 2*(k%4) (least significant first): 0 = backbone
      -alpha, 1 = zero, 2 = backbone +alpha, 3 = residual;
  residual stream [N][ld] int8: the codes of R in increasing k, then zeros;
      ld is a multiple of 16 that no row's residual count can exceed.
"""
from __future__ import annotations

import numpy as np

from .numerics import exact_abs_sum_units, round_rational_to_f32
from .quant import absmax_scale, quantize_with_scale

FIELD_NEG, FIELD_ZERO, FIELD_POS, FIELD_RES = 0, 1, 2, 3


def nearest_rank(pct: int, k: int) -> int:
    """j = ceil(pct * k / 100) in exact integer arithmetic (0 for pct = 0)."""
    if not 0 <= pct <= 100:
        raise ValueError("percentile must be in 0..100")
    return (pct * k + 99) // 100


def check_percentiles(pct_backbone: int, pct_zero: int):
    if not (1 <= pct_backbone <= 100 and 0 <= pct_zero <= pct_backbone):
        raise ValueError("need 1 <= pct_backbone <= 100 and 0 <= pct_zero <= pct_backbone")


def resid_ld(k: int, pct_zero: int) -> int:
    """Row stride of the residual stream: a multiple of 16 bytes covering the
    largest residual count a row can have.  At least j(P_z) magnitudes are
    <= eps, so |R| <= k - j(P_z)."""
    return ((k - nearest_rank(pct_zero, k)) + 15) // 16 * 16


def row_thresholds(w_row: np.ndarray, pct_backbone: int, pct_zero: int):
    """(tau, eps) of one row as fp32 magnitudes; eps is None for pct_zero = 0."""
    a = np.sort(np.abs(np.asarray(w_row, dtype=np.float32)))
    k = a.size
    tau = a[nearest_rank(pct_backbone, k) - 1]
    eps = a[nearest_rank(pct_zero, k) - 1] if pct_zero > 0 else None
    return np.float32(tau), (None if eps is None else np.float32(eps))


def threshold_split(w: np.ndarray, pct_backbone: int = 80, pct_zero: int = 50):
    """Per-row thresholded split of W [N][K] (fp32).

    Returns (fields uint8 [N][K] in 0..3, alpha fp32 [N], rq int8 [N][K]
    (the residual codes in place, 0 outside R), s_r fp32 [N])."""
    check_percentiles(pct_backbone, pct_zero)
    w = np.asarray(w, dtype=np.float32)
    if w.ndim != 2:
        raise ValueError("2-D weight expected")
    n, k = w.shape
    fields = np.empty((n, k), np.uint8)
    alpha = np.zeros(n, np.float32)
    s_r = np.ones(n, np.float32)
    rq = np.zeros((n, k), np.int8)
    for r in range(n):
        row = w[r]
        mag = np.abs(row)
        tau, eps = row_thresholds(row, pct_backbone, pct_zero)
        in_b = mag > tau
        in_z = (mag <= eps) if eps is not None else np.zeros(k, bool)
        in_r = ~in_b & ~in_z
        f = np.full(k, FIELD_ZERO, np.uint8)
        f[in_b & (row > 0)] = FIELD_POS
        f[in_b & (row < 0)] = FIELD_NEG
        f[in_r] = FIELD_RES
        fields[r] = f
        nb = int(in_b.sum())
        if nb:
            alpha[r] = round_rational_to_f32(exact_abs_sum_units(row[in_b]), nb << 149)
        if in_r.any():
            s = absmax_scale(np.array([mag[in_r].max()], np.float32))[0]
            s_r[r] = s
            rq[r, in_r] = quantize_with_scale(row[in_r], s)
    return fields, alpha, rq, s_r


def pack_threshold(fields: np.ndarray, rq: np.ndarray, ld: int):
    """-> (class plane uint8 [N][K/4], residual stream int8 [N][ld])."""
    fields = np.asarray(fields, np.uint8)
    n, k = fields.shape
    if k % 4 or fields.max(initial=0) > 3:
        raise ValueError("k % 4 == 0 and 2-bit fields expected")
    f = fields.reshape(n, k // 4, 4).astype(np.uint32)
    plane = (f[..., 0] | (f[..., 1] << 2) | (f[..., 2] << 4) | (f[..., 3] << 6)).astype(np.uint8)
    stream = np.zeros((n, ld), np.int8)
    for r in range(n):
        vals = np.asarray(rq[r])[fields[r] == FIELD_RES]
        if vals.size > ld:
            raise ValueError("residual count exceeds the row stride")
        stream[r, :vals.size] = vals
    return plane, stream


def unpack_threshold(plane: np.ndarray, stream: np.ndarray, k: int):
    """Inverse of pack_threshold -> (fields [N][K], rq [N][K] in place)."""
    plane = np.asarray(plane, np.uint8)
    n = plane.shape[0]
    fields = np.stack([(plane >> (2 * i)) & 3 for i in range(4)], axis=2).reshape(n, -1)[:, :k]
    rq = np.zeros((n, k), np.int8)
    for r in range(n):
        pos = np.nonzero(fields[r] == FIELD_RES)[0]
        rq[r, pos] = np.asarray(stream[r, :pos.size], np.int8)
    return fields.astype(np.uint8), rq


def int_products(fields: np.ndarray, rq: np.ndarray, xq: np.ndarray):
    """(acc_b, acc_r) int64 [N]: acc_b = sum of x_q over backbone +alpha
    weights minus the sum over backbone -alpha weights; acc_r = sum_R q x_q.
    Exact (fp64 on integer values: |partial sums| <= K * 127 * 127 < 2**53)."""
    fields = np.asarray(fields)
    x = np.asarray(xq, np.float64).ravel()
    if fields.shape[1] * 127 * 127 >= 2 ** 53:
        raise OverflowError("fp64 product would not be exact")
    sgn = np.where(fields == FIELD_POS, 1.0, np.where(fields == FIELD_NEG, -1.0, 0.0))
    acc_b = sgn @ x
    acc_r = np.asarray(rq, np.float64) @ x
    return acc_b.astype(np.int64), acc_r.astype(np.int64)


def y_threshold(acc_b, acc_r, alpha, s_r, s_x, skip_residual: bool = False) -> np.ndarray:
    """y = alpha * acc_b / s_x + acc_r / (s_r * s_x) in fp64; with
    skip_residual only the backbone term ([SEP] section 3.3 fast mode)."""
    sx = np.float64(np.asarray(s_x).ravel()[0])
    y = np.asarray(alpha, np.float64) * np.asarray(acc_b, np.float64) / sx
    if not skip_residual:
        y = y + np.asarray(acc_r, np.float64) / (np.asarray(s_r, np.float64) * sx)
    return y


def dequantize_threshold(fields, alpha, rq, s_r) -> np.ndarray:
    """W_hat [N][K] in fp64: +-alpha on B, q / s_r on R, 0 on Z."""
    fields = np.asarray(fields)
    a = np.asarray(alpha, np.float64)[:, None]
    sgn = np.where(fields == FIELD_POS, 1.0, np.where(fields == FIELD_NEG, -1.0, 0.0))
    return a * sgn + np.asarray(rq, np.float64) / np.asarray(s_r, np.float64)[:, None]
