"""MXFP4 block-scaled 4-bit floating point for the format-separated prefill
(oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[DQ] (quantization split by inference phase): "format separation" runs the prefill on the accelerator's native low-bit
quantized compute (NVFP4 on the hardware the page measures) while decode
keeps a low-bit weight-only format; the prefill speed-up comes from that
native compute.  The native 4-bit block format of this library's matrix
cores is OCP microscaling MXFP4, which this module defines (the pages do not
give NVFP4's or MXFP4's encoding; this is the reading):

  * a block is 32 consecutive values of a row (along K);
  * its shared scale is X = 2**e with e = floor(log2(max |v|)) - 2 (2 is the
    largest exponent of the element format, whose largest value is
    6 = 1.5 * 2**2), clamped to [-127, 127], stored as the E8M0 byte e + 127;
    an all-zero block has e = 0;
  * each element is the E2M1 value nearest to v / X (exact: X is a power of
    two), ties to the even code, magnitudes above 6 saturating to 6.  E2M1
    magnitudes are {0, 0.5, 1, 1.5, 2, 3, 4, 6} for codes 0..7; bit 3 is the
    sign, set for v < 0 (so -0.0 encodes as +0);
  * storage (this library's layout, K % 256 == 0): codes [R][K/2] bytes,
    element 2j of a row in the low nibble of byte j; scales [K/256][R][8]
    E8M0 bytes -- the 8 block scales of 256 consecutive values of a row
    together, and those of all rows for one 256-value slice of K together
    (the slices a GEMM stages).
The product of two quantized operands is sum_k a[m][k] * b[n][k] with each
operand value = E2M1 value * 2**e of its block (fp64 here).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E2M1 = np.array([0.0, 0.5, 1.0, 1.5, 2.0, 3.0, 4.0, 6.0], np.float64)
EMAX_ELEM = 2


def e2m1_round(a: np.ndarray) -> np.ndarray:
    """Magnitude code 0..7 of |value| a >= 0: nearest E2M1 value, ties to the
    even code, saturating at 6 (brute force over the 8 values; large inputs
    are taken a slice at a time to bound memory)."""
    a = np.asarray(a, np.float64)
    if a.size > (1 << 20):
        flat = a.ravel()
        out = np.empty(flat.size, np.uint8)
        for lo in range(0, flat.size, 1 << 20):
            out[lo:lo + (1 << 20)] = e2m1_round(flat[lo:lo + (1 << 20)])
        return out.reshape(a.shape)
    a = np.minimum(a, 6.0)
    d = np.abs(a[..., None] - E2M1)                       # distance to every value
    best = d.min(axis=-1, keepdims=True)
    cand = d == best                                       # nearest (one or two)
    codes = np.arange(8)
    even_pick = np.where(cand & (codes % 2 == 0), codes, 99).min(axis=-1)
    any_pick = np.where(cand, codes, 99).min(axis=-1)
    two = cand.sum(axis=-1) > 1
    return np.where(two, even_pick, any_pick).astype(np.uint8)


def block_exponent(amax: np.ndarray) -> np.ndarray:
    """e = floor(log2(amax)) - 2, clamped to [-127, 127]; 0 for amax = 0.
    floor(log2) of an fp32 value is read off its exponent bits (exact)."""
    a = np.asarray(amax, np.float32)
    _, ex = np.frexp(a.astype(np.float64))               # a = f * 2**ex, f in [0.5, 1)
    e = ex.astype(np.int64) - 1 - EMAX_ELEM
    e = np.clip(e, -127, 127)
    return np.where(a == 0, 0, e).astype(np.int64)


def quantize_mxfp4(x: np.ndarray):
    """x [R][K] (fp32 values; K % 32 == 0) -> (codes uint8 [R][K] in 0..15,
    exponents int64 [R][K/32])."""
    x = np.asarray(x, np.float32)
    r, k = x.shape
    if k % BLOCK:
        raise ValueError("K must be a multiple of 32")
    blk = x.reshape(r, k // BLOCK, BLOCK)
    amax = np.abs(blk).max(axis=2)
    e = block_exponent(amax)
    scaled = blk.astype(np.float64) / np.ldexp(1.0, e)[..., None]   # exact
    mag = e2m1_round(np.abs(scaled))
    sign = (blk < 0).astype(np.uint8)
    codes = (sign << 3) | mag
    return codes.reshape(r, k).astype(np.uint8), e


def dequantize_mxfp4(codes, e) -> np.ndarray:
    """Values (fp64) of MXFP4 codes [R][K] with block exponents [R][K/32]."""
    codes = np.asarray(codes, np.uint8)
    r, k = codes.shape
    mag = E2M1[codes & 7]
    val = np.where(codes & 8, -mag, mag)
    return val * np.repeat(np.ldexp(1.0, np.asarray(e)), BLOCK, axis=1)


def pack_mxfp4(codes, e):
    """-> (packed codes uint8 [R][K/2], E8M0 scales uint8 [K/256][R][8])."""
    codes = np.asarray(codes, np.uint8)
    r, k = codes.shape
    if k % 256:
        raise ValueError("K must be a multiple of 256")
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sc = (np.asarray(e) + 127).astype(np.uint8).reshape(r, k // 256, 8)
    return packed, np.ascontiguousarray(sc.transpose(1, 0, 2))


def unpack_mxfp4(packed, scales):
    packed = np.asarray(packed, np.uint8)
    r, h = packed.shape
    codes = np.empty((r, 2 * h), np.uint8)
    codes[:, 0::2] = packed & 15
    codes[:, 1::2] = packed >> 4
    sc = np.asarray(scales, np.int64).transpose(1, 0, 2).reshape(r, -1)
    return codes, sc - 127


def gemm_mxfp4(ca, ea, cb, eb) -> np.ndarray:
    """Y[m][n] = sum_k A[m][k] B[n][k] of two MXFP4 operands, fp64."""
    return dequantize_mxfp4(ca, ea) @ dequantize_mxfp4(cb, eb).T
