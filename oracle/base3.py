"""Base-3 packing of ternary codes, five to a byte (test infrastructure only).

[VG] 'BitNet b1.58': a weight with three states carries log2(3) ~ 1.58 bits,
so 2-bit fields waste 0.42 bit per weight.  Since 3**5 = 243 <= 256, five
ternary digits fit in one byte: 1.6 bits per weight.  The pages give no
layout; this library's is:

* digit f = q + 1 in {0, 1, 2} for a code q in {-1, 0, 1};
* weights 5j .. 5j+4 of a row form the base-3 number
  v = sum_{i<5} f[5j+i] * 3**(4-i) (the first weight is the leading digit),
  0 <= v <= 242;
* the stored byte is t = ceil(256 * v / 243): the base-3 fraction v / 243
  rounded up to 8 bits.  Multiplying by 3 then moves the next digit into the
  integer part: digit i = (3 * t_i) >> 8 and t_{i+1} = (3 * t_i) mod 256.  This
  is exact because rounding up adds less than 1/256 < 1/243 to the fraction,
  which never reaches the next multiple of 3**-(5-i) after i steps;
* a row takes 16 * ceil(k / 80) bytes (80 weights per 16-byte chunk); the
  weights past k are digit 1 (q = 0).
"""
from __future__ import annotations

import numpy as np

PER_BYTE = 5
PER_CHUNK = 80  # weights per 16-byte chunk


def row_bytes(k: int) -> int:
    """Bytes of one packed row: 16 per 80 weights, rounded up."""
    return 16 * ((k + PER_CHUNK - 1) // PER_CHUNK)


def encode_digits(digits) -> int:
    """Byte of five base-3 digits (leading digit first)."""
    v = 0
    for f in digits:
        if f not in (0, 1, 2):
            raise ValueError("digit out of range")
        v = 3 * v + f
    return (256 * v + 242) // 243  # ceil(256 v / 243)


def decode_byte(t: int):
    """Five digits of a stored byte, by repeated multiplication by 3."""
    out = []
    for _ in range(PER_BYTE):
        m = 3 * t
        out.append(m >> 8)
        t = m & 255
    return out


def _digits(codes: np.ndarray) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int8).astype(np.int16)
    if np.any((c < -1) | (c > 1)):
        raise ValueError("ternary codes must be in {-1, 0, 1}")
    return (c + 1).astype(np.int64)


def pack_base3(codes: np.ndarray) -> np.ndarray:
    """[n][k] int8 codes -> [n][row_bytes(k)] uint8 (vectorized)."""
    codes = np.atleast_2d(np.asarray(codes))
    n, k = codes.shape
    nb = row_bytes(k)
    f = np.ones((n, nb * PER_BYTE), np.int64)  # padding digit 1 (q = 0)
    f[:, :k] = _digits(codes)
    f = f.reshape(n, nb, PER_BYTE)
    v = np.zeros((n, nb), np.int64)
    for i in range(PER_BYTE):
        v = 3 * v + f[:, :, i]
    return ((256 * v + 242) // 243).astype(np.uint8)


def unpack_base3(packed: np.ndarray, k: int) -> np.ndarray:
    """Inverse of pack_base3: [n][row_bytes(k)] uint8 -> [n][k] int8 codes."""
    t = np.atleast_2d(np.asarray(packed, dtype=np.uint8)).astype(np.int64)
    n, nb = t.shape
    f = np.empty((n, nb, PER_BYTE), np.int64)
    for i in range(PER_BYTE):
        m = 3 * t
        f[:, :, i] = m >> 8
        t = m & 255
    return (f.reshape(n, -1)[:, :k] - 1).astype(np.int8)


def pack_base3_loops(codes):
    """The same layout with explicit loops over bytes and digits (small inputs)."""
    rows = [list(map(int, r)) for r in np.atleast_2d(np.asarray(codes))]
    out = []
    for row in rows:
        k = len(row)
        nb = row_bytes(k)
        padded = [q + 1 for q in row] + [1] * (nb * PER_BYTE - k)
        out.append([encode_digits(padded[PER_BYTE * j:PER_BYTE * j + PER_BYTE]) for j in range(nb)])
    return np.array(out, dtype=np.uint8)


def unpack_base3_loops(packed, k: int):
    out = []
    for prow in np.atleast_2d(np.asarray(packed, dtype=np.uint8)):
        digits = []
        for t in prow:
            digits.extend(decode_byte(int(t)))
        out.append([d - 1 for d in digits[:k]])
    return np.array(out, dtype=np.int8)
