"""Group-wise 4-bit weights with zero-points and two-level scales (oracle).

TEST INFRASTRUCTURE ONLY (see the package docstring).

[VG] 'Why Q4_K splits weights into blocks' and 'Q4_K uses two-level blocks'
(figs. 43-46): the weights of a row are split along the summed dimension
into super-blocks of 256, each of 8 groups of 32.  A group maps its weights
asymmetrically onto 0..15 with its own scale and minimum,
    q = clip(round((w - min) / scale), 0, 15),   w_hat = q * scale + min,
and the 8 group scales and minimums are themselves quantized to 6 bits
against two fp16 super-block factors d and dmin ('the scales are quantized
too'), which makes 144 bytes per 256 weights, 4.5 bits per weight.

Readings where the page leaves the procedure open:
  * a group's scale is (max - min) / 15 and its minimum is its min (fp32);
  * d = fp16(max_j scale_j / 63), sc_j = clip(rne(scale_j / d), 0, 63);
  * minimums keep their sign: dmin = fp16(max_j |min_j| / 31),
    m_j = clip(rne(min_j / dmin), -31, 31), stored biased as m_j + 32;
  * the 4-bit codes are taken against the reconstructed S_j = d * sc_j and
    M_j = dmin * m_j (both exact in fp32), so that w_hat = q * S_j + M_j is
    what the stored bytes mean; S_j = 0 gives codes 0;
  * rounding is half-to-even, fp32 arithmetic in the order written, fp16 by
    round-to-nearest-even.

Storage (this library's own layout, planar so that a GPU streams it with
16-byte loads):
  codes [N][K/2] bytes: weight k of a row in byte k/2, low nibble first;
  meta  [N][K/256][16] bytes per super-block: bytes 0-11 hold sixteen 6-bit
        fields, LSB first (field i at bits 6i..6i+5 of the little-endian
        96-bit value): sc_0..sc_7 then m_0+32..m_7+32; bytes 12-13 d and
        14-15 dmin as little-endian fp16 bit patterns.
"""
from __future__ import annotations

import numpy as np

from .numerics import bf16_bits_to_f32

GROUP = 32
SUPER = 256
GROUPS_PER_SUPER = SUPER // GROUP
META_BYTES = 16


def group_params(w_group: np.ndarray):
    """Level 1: (scale, min) of one group, fp32 ('Why Q4_K splits weights
    into blocks': each block keeps its own scale and minimum)."""
    g = np.asarray(w_group, dtype=np.float32)
    lo = np.float32(np.min(g))
    hi = np.float32(np.max(g))
    scale = np.float32(np.float32(hi - lo) / np.float32(15))
    return scale, lo


def quantize_q4k(w: np.ndarray):
    """Two-level quantization of W [N][K] (K % 256 == 0), every group at once
    (the same fp32 operations as group_params and the readings above).
    Returns (codes uint8 [N][K] in 0..15, sc uint8 [N][K/32] in 0..63,
    m int8 [N][K/32] in -31..31, d fp16 [N][K/256], dmin fp16 [N][K/256])."""
    w = np.asarray(w, dtype=np.float32)
    n, k = w.shape
    if k % SUPER:
        raise ValueError("K must be a multiple of 256")
    f32 = np.float32
    g = w.reshape(n, k // SUPER, GROUPS_PER_SUPER, GROUP)        # [row][super-block][group][32]
    lo = g.min(axis=3)
    hi = g.max(axis=3)
    scale = ((hi - lo).astype(f32) / f32(15)).astype(f32)         # level 1: per group
    d = (scale.max(axis=2) / f32(63)).astype(f32).astype(np.float16)          # level 2: per super-block
    dmin = (np.abs(lo).max(axis=2) / f32(31)).astype(f32).astype(np.float16)
    d32 = d.astype(f32)[..., None]
    dm32 = dmin.astype(f32)[..., None]
    with np.errstate(divide="ignore", invalid="ignore"):
        sc = np.where(d32 == 0, f32(0), np.clip(np.rint((scale / d32).astype(f32)), 0, 63)).astype(f32)
        mm = np.where(dm32 == 0, f32(0), np.clip(np.rint((lo / dm32).astype(f32)), -31, 31)).astype(f32)
        S = (d32 * sc).astype(f32)[..., None]
        M = (dm32 * mm).astype(f32)[..., None]
        q = np.where(S == 0, f32(0), np.clip(np.rint(((g - M).astype(f32) / S).astype(f32)), 0, 15))
    codes = q.astype(np.uint8).reshape(n, k)
    return (codes, sc.astype(np.uint8).reshape(n, -1), mm.astype(np.int8).reshape(n, -1), d, dmin)


def reconstructed_params(sc, mm, d, dmin):
    """S [N][K/32] = d * sc and M [N][K/32] = dmin * m, exact in fp32."""
    d32 = np.repeat(np.asarray(d, np.float32), GROUPS_PER_SUPER, axis=1)
    dm32 = np.repeat(np.asarray(dmin, np.float32), GROUPS_PER_SUPER, axis=1)
    S = (d32 * np.asarray(sc, np.float32)).astype(np.float32)
    M = (dm32 * np.asarray(mm, np.float32)).astype(np.float32)
    return S, M


def dequantize_q4k(codes, sc, mm, d, dmin) -> np.ndarray:
    """w_hat = q * S + M, in fp64 (exact)."""
    S, M = reconstructed_params(sc, mm, d, dmin)
    S64 = np.repeat(S.astype(np.float64), GROUP, axis=1)
    M64 = np.repeat(M.astype(np.float64), GROUP, axis=1)
    return np.asarray(codes, np.float64) * S64 + M64


def pack_fields6(vals) -> bytes:
    """Sixteen 6-bit values -> 12 bytes, LSB first."""
    acc = 0
    for i, v in enumerate(vals):
        if not 0 <= int(v) < 64:
            raise ValueError("6-bit field out of range")
        acc |= int(v) << (6 * i)
    return acc.to_bytes(12, "little")


def unpack_fields6(b: bytes):
    acc = int.from_bytes(bytes(b), "little")
    return [(acc >> (6 * i)) & 63 for i in range(16)]


def pack_q4k(codes, sc, mm, d, dmin):
    """-> (codes plane uint8 [N][K/2], meta plane uint8 [N][K/256][16])."""
    codes = np.asarray(codes, np.uint8)
    n, k = codes.shape
    if codes.max(initial=0) > 15:
        raise ValueError("4-bit codes expected")
    plane = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    ns = k // SUPER
    fields = np.concatenate([np.asarray(sc, np.int64).reshape(n, ns, 8),
                             np.asarray(mm, np.int64).reshape(n, ns, 8) + 32], axis=2)    # [n][ns][16]
    if fields.min(initial=0) < 0 or fields.max(initial=0) > 63:
        raise ValueError("6-bit field out of range")
    bits = ((fields[..., None] >> np.arange(6)) & 1).astype(np.uint8).reshape(n, ns, 96)   # field i -> bits 6i..
    meta = np.zeros((n, ns, META_BYTES), np.uint8)
    meta[..., :12] = np.packbits(bits, axis=2, bitorder="little")
    meta[..., 12:14] = np.asarray(d, np.float16).view(np.uint16)[..., None].view(np.uint8).reshape(n, ns, 2)
    meta[..., 14:16] = np.asarray(dmin, np.float16).view(np.uint16)[..., None].view(np.uint8).reshape(n, ns, 2)
    return plane, meta


def unpack_q4k(plane, meta):
    """Inverse of pack_q4k -> (codes, sc, mm, d, dmin)."""
    plane = np.asarray(plane, np.uint8)
    meta = np.asarray(meta, np.uint8)
    n, half = plane.shape
    codes = np.zeros((n, 2 * half), np.uint8)
    codes[:, 0::2] = plane & 15
    codes[:, 1::2] = plane >> 4
    ns = meta.shape[1]
    bits = np.unpackbits(meta[..., :12], axis=2, bitorder="little").reshape(n, ns, 16, 6).astype(np.int64)
    fields = (bits << np.arange(6)).sum(axis=3)
    sc = fields[..., :8].reshape(n, -1).astype(np.uint8)
    mm = (fields[..., 8:] - 32).reshape(n, -1).astype(np.int8)
    d = np.ascontiguousarray(meta[..., 12:14]).view(np.uint16)[..., 0].view(np.float16)
    dmin = np.ascontiguousarray(meta[..., 14:16]).view(np.uint16)[..., 0].view(np.float16)
    return codes, sc, mm, d, dmin


def y_q4k(codes, sc, mm, d, dmin, x_bf16_bits) -> np.ndarray:
    """y[n] = sum_k w_hat[n][k] x[k] in fp64 (x given as bf16 bits)."""
    x = bf16_bits_to_f32(np.asarray(x_bf16_bits, np.uint16)).astype(np.float64)
    return dequantize_q4k(codes, sc, mm, d, dmin) @ x
