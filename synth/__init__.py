"""Seeded synthetic inputs for the quantized-GEMV workloads.

This module only draws random tensors of the shapes and value distributions
that the quantization pages describe (LLM weights "roughly Gaussian or
Laplace" with a few large entries; activations with a handful of channels
tens of times larger than the rest).  It holds none of the method's
arithmetic: no scales, no rounding to integer codes, no packing, no products.
Both the CPU oracle's tests and the GPU path's tests/bench draw from here, so
the two sides always see the same bytes.

Conventions
-----------
* RNG: ``numpy.random.Generator(PCG64(seed))``.
* Draw order inside one workload: W, then W's outlier mask, then x (or X),
  then the outlier channel indices of X.
* "p% of entries x c": a Bernoulli(p) mask drawn with ``rng.random(shape)``.
* bf16 tensors are drawn in fp32 and narrowed to bf16 by round-to-nearest-even
  on the fp32 bit pattern; they are returned as ``uint16`` bit patterns.
"""
from __future__ import annotations

from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np


def rng(seed: int) -> np.random.Generator:
    return np.random.Generator(np.random.PCG64(seed))


def to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Narrow fp32 values to bf16 bit patterns (round to nearest, ties even).

    Input data type conversion only (finite inputs)."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (b >> np.uint64(16)) & np.uint64(1)
    r = (b + np.uint64(0x7FFF) + lsb) >> np.uint64(16)
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << np.uint32(16)).view(np.float32)


def gaussian(g: np.random.Generator, shape, std: float) -> np.ndarray:
    return (g.standard_normal(shape, dtype=np.float64) * std).astype(np.float32)


def laplace(g: np.random.Generator, shape, b: float) -> np.ndarray:
    return g.laplace(0.0, b, size=shape).astype(np.float32)


def boost_entries(g: np.random.Generator, w: np.ndarray, p: float, factor: float) -> int:
    """Multiply a Bernoulli(p) subset of w's entries by `factor` in place;
    returns the realised count."""
    mask = g.random(w.shape) < p
    w[mask] *= np.float32(factor)
    return int(mask.sum())


@dataclass
class Workload:
    name: str
    seed: int
    tensors: Dict[str, np.ndarray] = field(default_factory=dict)
    meta: Dict[str, object] = field(default_factory=dict)


# --------------------------------------------------------------------------
# The five workloads.  Sizes can be overridden (smaller shapes with the same
# distributions are what the CPU-sized parity tests use).
# --------------------------------------------------------------------------

def tiny_gemv(n: int = 256, k: int = 256, seed: int = 1) -> Workload:
    """W fp32 [n][k] ~ N(0, 0.02); x fp32 [k] ~ N(0, 1)."""
    g = rng(seed)
    w = gaussian(g, (n, k), 0.02)
    x = gaussian(g, (k,), 1.0)
    return Workload("tiny_w8a8", seed, {"w": w, "x": x}, {"n": n, "k": k})


DECODE_7B_SHAPES = {  # (N, K) of one 4096-hidden / 11008-FFN layer's projections
    "attn_4096x4096": (4096, 4096),
    "ffn_up_11008x4096": (11008, 4096),
    "ffn_down_4096x11008": (4096, 11008),
}
DECODE_7B_SEEDS = {"attn_4096x4096": 21, "ffn_up_11008x4096": 22, "ffn_down_4096x11008": 23}


def decode_w8a16(n: int = 4096, k: int = 4096, seed: int = 21) -> Workload:
    """W ~ N(0, 0.02) with 0.1% of entries x10; x bf16 ~ N(0, 1)."""
    g = rng(seed)
    w = gaussian(g, (n, k), 0.02)
    cnt = boost_entries(g, w, 0.001, 10.0)
    x = to_bf16_bits(gaussian(g, (k,), 1.0))
    return Workload("decode_w8a16", seed, {"w": w, "x_bf16": x},
                    {"n": n, "k": k, "boosted": cnt})


def ternary_decode(n: int = 11008, k: int = 4096, seed: int = 3) -> Workload:
    """W ~ Laplace(0, 0.02); x fp32 ~ N(0, 1)."""
    g = rng(seed)
    w = laplace(g, (n, k), 0.02)
    x = gaussian(g, (k,), 1.0)
    return Workload("ternary_decode", seed, {"w": w, "x": x}, {"n": n, "k": k})


def sign_residual_decode(n: int = 28672, k: int = 8192, seed: int = 4,
                         rows: Optional[np.ndarray] = None) -> Workload:
    """W ~ Laplace(0, 0.015) with 0.5% of entries x20; x bf16 ~ N(0, 1).

    With `rows` given, the full [n][k] matrix is still drawn (so the bytes
    equal those of the full workload) but only those rows are returned."""
    g = rng(seed)
    w = laplace(g, (n, k), 0.015)
    cnt = boost_entries(g, w, 0.005, 20.0)
    x = to_bf16_bits(gaussian(g, (k,), 1.0))
    if rows is not None:
        w = np.ascontiguousarray(w[rows])
    return Workload("sign_residual_decode", seed, {"w": w, "x_bf16": x},
                    {"n": n, "k": k, "boosted": cnt})


def prefill_outlier(m: int = 2048, k: int = 4096, n: int = 4096, n_out: int = 20,
                    seed: int = 5) -> Workload:
    """W [n][k] ~ N(0, 0.02); X bf16 [m][k] ~ N(0, 1) with `n_out` seed-chosen
    channels scaled x50 before narrowing to bf16; idx sorted int32."""
    g = rng(seed)
    w = gaussian(g, (n, k), 0.02)
    x = gaussian(g, (m, k), 1.0)
    idx = np.sort(g.choice(k, size=n_out, replace=False)).astype(np.int32)
    x[:, idx] *= np.float32(50.0)
    return Workload("prefill_w8a8_outlier", seed,
                    {"w": w, "x_bf16": to_bf16_bits(x), "idx": idx},
                    {"m": m, "k": k, "n": n, "n_out": n_out})


def q4_decode(n: int = 11008, k: int = 4096, seed: int = 6) -> Workload:
    """Group-wise 4-bit decode at the 7B FFN shape: W ~ N(0, 0.02) with 0.1%
    of entries x10 (the W8A16 decode recipe); x bf16 ~ N(0, 1)."""
    g = rng(seed)
    w = gaussian(g, (n, k), 0.02)
    cnt = boost_entries(g, w, 0.001, 10.0)
    x = to_bf16_bits(gaussian(g, (k,), 1.0))
    return Workload("q4_decode", seed, {"w": w, "x_bf16": x}, {"n": n, "k": k, "boosted": cnt})
