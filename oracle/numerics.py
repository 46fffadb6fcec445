"""Number-format helpers of the oracle (test infrastructure only).

* bf16 <-> fp32 by definition: bf16 is the top half of the fp32 bit pattern;
  narrowing rounds to nearest, ties to even ([OVR] section 4, data-type table:
  bf16 keeps fp32's 8 exponent bits and 7 mantissa bits).
* Correct rounding of an exact rational to fp32 (round to nearest, ties to
  even, subnormals included).
* Exact sums of |x| over fp32 values, and the correctly rounded mean of |x|
  that the absmean and sign-backbone scales are defined from.
"""
from __future__ import annotations

import math

import numpy as np

_FLT_MAX_EXP_ULP = 104  # FLT_MAX = (2**24 - 1) * 2**104


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    """bf16 bit patterns (uint16) -> exact fp32 values."""
    h = np.ascontiguousarray(h, dtype=np.uint16)
    return (h.astype(np.uint32) << np.uint32(16)).view(np.float32)


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """fp32 -> bf16 bit patterns, round to nearest with ties to even on the
    16 discarded bits (finite inputs)."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep = u >> np.uint64(16)
    low = u & np.uint64(0xFFFF)
    up = (low > np.uint64(0x8000)) | ((low == np.uint64(0x8000)) & ((keep & np.uint64(1)) == np.uint64(1)))
    return (keep + up.astype(np.uint64)).astype(np.uint16)


def round_rational_to_f32(num: int, den: int) -> np.float32:
    """The fp32 value nearest to num/den (num >= 0, den > 0), ties to even.

    Written from the definition of IEEE binary32: 24-bit significands for
    normal numbers, a fixed quantum of 2**-149 below 2**-126."""
    if den <= 0 or num < 0:
        raise ValueError("need num >= 0 and den > 0")
    if num == 0:
        return np.float32(0.0)
    e = num.bit_length() - den.bit_length()
    if (num < (den << e)) if e >= 0 else ((num << -e) < den):
        e -= 1
    # now 2**e <= num/den < 2**(e+1)
    ulp_e = max(e, -126) - 23
    if ulp_e >= 0:
        n2, d2 = num, den << ulp_e
    else:
        n2, d2 = num << -ulp_e, den
    q, r = divmod(n2, d2)
    if 2 * r > d2 or (2 * r == d2 and (q & 1)):
        q += 1
    if ulp_e > _FLT_MAX_EXP_ULP or (ulp_e == _FLT_MAX_EXP_ULP and q >= (1 << 24)):
        raise OverflowError("value exceeds FLT_MAX")
    return np.float32(math.ldexp(q, ulp_e))


def _abs_units(a: np.ndarray):
    """Split |a| (fp32) into integer significands and shifts such that
    |a_i| = mant_i * 2**(shift_i - 149) exactly."""
    bits = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32) & np.uint32(0x7FFFFFFF)
    if np.any((bits >> np.uint32(23)) == np.uint32(255)):
        raise ValueError("non-finite input")
    e = (bits >> np.uint32(23)).astype(np.int64)
    mant = (bits & np.uint32(0x7FFFFF)).astype(np.int64) | np.where(e > 0, 1 << 23, 0)
    shift = np.maximum(e, 1) - 1
    return mant, shift


def exact_abs_sum_units(a: np.ndarray) -> int:
    """Exact integer S with sum_i |a_i| = S * 2**-149 (a: fp32, any shape).

    Significands are summed per binade with numpy (each binade's sum is an
    integer below 2**53 per chunk, hence exact in fp64), then the binades
    are combined with Python's unbounded integers."""
    flat = np.ascontiguousarray(a, dtype=np.float32).ravel()
    total = 0
    chunk = 1 << 28  # chunk * 2**24 < 2**53 keeps every partial sum exact
    for lo in range(0, flat.size, chunk):
        mant, shift = _abs_units(flat[lo:lo + chunk])
        sums = np.bincount(shift, weights=mant.astype(np.float64), minlength=1)
        for sh in np.nonzero(sums)[0]:
            total += int(sums[sh]) << int(sh)
    return total


def mean_abs_f32(a: np.ndarray) -> np.float32:
    """fp32 nearest to the exact mean of |a| (ties to even).

    The absmean scale of [VG] 'BitNet b1.58' (Fig. 60) and the mean-|W|
    scale of [VG] 'BitNet, weight quantization' (Fig. 55) are the average
    absolute weight; this is that real number, rounded once."""
    n = int(np.asarray(a).size)
    if n == 0:
        raise ValueError("empty")
    return round_rational_to_f32(exact_abs_sum_units(a), n << 149)


def mean_abs_rows_f32(w: np.ndarray) -> np.ndarray:
    """Per-row mean_abs_f32 of a 2-D fp32 array."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    n, k = w.shape
    out = np.empty(n, dtype=np.float32)
    rows_per_block = max(1, (1 << 24) // max(k, 1))
    for r0 in range(0, n, rows_per_block):
        blk = w[r0:r0 + rows_per_block]
        nb = blk.shape[0]
        mant, shift = _abs_units(blk)
        key = (np.arange(nb, dtype=np.int64)[:, None] * 256 + shift).ravel()
        sums = np.bincount(key, weights=mant.ravel().astype(np.float64), minlength=nb * 256)
        sums = sums.reshape(nb, 256)
        for i in range(nb):
            s = 0
            for sh in np.nonzero(sums[i])[0]:
                s += int(sums[i, sh]) << int(sh)
            out[r0 + i] = round_rational_to_f32(s, k << 149)
    return out
