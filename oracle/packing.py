"""Bit packing of low-bit codes (test infrastructure only).

Storage cost per weight is the point of the low-bit formats ([SEP] section
3.2: a 1-bit backbone costs 0.125 byte per weight; [VG] 'BitNet b1.58':
three states carry log2(3) ~ 1.58 bits).  The pages fix no bit order, so the
layout is the plainest one:

* bits = 2 (ternary): field = q + 1 in {0, 1, 2}; 4 fields per byte.
* bits = 1 (sign):    field = 1 for +1, 0 for -1;   8 fields per byte.
* Code k of a row lives in byte k // v at bit offset bits * (k % v), least
  significant field first (v = 8 // bits); rows are contiguous, row-major.
"""
from __future__ import annotations

import numpy as np


def _fields(codes: np.ndarray, bits: int) -> np.ndarray:
    c = np.asarray(codes, dtype=np.int8).astype(np.int16)
    if bits == 2:
        if np.any((c < -1) | (c > 1)):
            raise ValueError("ternary codes must be in {-1, 0, 1}")
        return (c + 1).astype(np.uint8)
    if bits == 1:
        if np.any((c != -1) & (c != 1)):
            raise ValueError("sign codes must be +-1")
        return (c == 1).astype(np.uint8)
    raise ValueError("bits must be 1 or 2")


def pack(codes: np.ndarray, bits: int) -> np.ndarray:
    """Vectorized packing; [n][k] int8 codes -> [n][k * bits / 8] uint8."""
    codes = np.asarray(codes)
    if codes.ndim == 1:
        codes = codes[None, :]
    n, k = codes.shape
    v = 8 // bits
    if k % v:
        raise ValueError("k must be a multiple of %d" % v)
    f = _fields(codes, bits).reshape(n, k // v, v).astype(np.uint32)
    shifts = (np.arange(v, dtype=np.uint32) * bits)[None, None, :]
    return np.bitwise_or.reduce(f << shifts, axis=2).astype(np.uint8)


def unpack(packed: np.ndarray, bits: int, k: int) -> np.ndarray:
    """Inverse of pack: [n][k * bits / 8] uint8 -> [n][k] int8 codes."""
    p = np.asarray(packed, dtype=np.uint8)
    if p.ndim == 1:
        p = p[None, :]
    n = p.shape[0]
    v = 8 // bits
    shifts = (np.arange(v, dtype=np.uint32) * bits)[None, None, :]
    f = (p.astype(np.uint32)[:, :, None] >> shifts) & np.uint32((1 << bits) - 1)
    f = f.reshape(n, -1)[:, :k].astype(np.int16)
    if bits == 2:
        return (f - 1).astype(np.int8)
    return np.where(f == 1, 1, -1).astype(np.int8)


def pack_loops(codes, bits: int):
    """The same layout with explicit Python loops (small inputs only)."""
    codes = [list(map(int, row)) for row in np.atleast_2d(np.asarray(codes))]
    v = 8 // bits
    out = []
    for row in codes:
        if len(row) % v:
            raise ValueError("ragged row")
        prow = []
        for b in range(len(row) // v):
            byte = 0
            for j in range(v):
                q = row[b * v + j]
                if bits == 2:
                    if q not in (-1, 0, 1):
                        raise ValueError("bad ternary code")
                    field = q + 1
                else:
                    if q not in (-1, 1):
                        raise ValueError("bad sign code")
                    field = 1 if q == 1 else 0
                byte |= field << (bits * j)
            prow.append(byte)
        out.append(prow)
    return np.array(out, dtype=np.uint8)


def unpack_loops(packed, bits: int, k: int):
    v = 8 // bits
    out = []
    for prow in np.atleast_2d(np.asarray(packed, dtype=np.uint8)):
        row = []
        for c in range(k):
            field = (int(prow[c // v]) >> (bits * (c % v))) & ((1 << bits) - 1)
            row.append(field - 1 if bits == 2 else (1 if field == 1 else -1))
        out.append(row)
    return np.array(out, dtype=np.int8)
