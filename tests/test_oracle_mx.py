"""Pins of the MXFP4 oracle: the E2M1 grid and its round-half-to-even rule,
the block-scale rule, exactness on representable blocks, the error bound,
packing, and the product against exact rationals."""
from fractions import Fraction

import numpy as np

import oracle.mx as mx
import synth


def test_grid_values_and_ties():
    for c, v in enumerate(mx.E2M1):
        assert mx.e2m1_round(np.array([v]))[0] == c
    ties = {0.25: 0, 0.75: 2, 1.25: 2, 1.75: 4, 2.5: 4, 3.5: 6, 5.0: 6}  # to the even code
    for v, c in ties.items():
        assert mx.e2m1_round(np.array([v]))[0] == c, v
        up = np.nextafter(v, np.inf)
        dn = np.nextafter(v, -np.inf)
        lo = int(np.max(np.nonzero(mx.E2M1 < v)[0]))
        assert mx.e2m1_round(np.array([up]))[0] == lo + 1 and mx.e2m1_round(np.array([dn]))[0] == lo
    for v in (6.0, 6.5, 7.999, 1e9):
        assert mx.e2m1_round(np.array([v]))[0] == 7  # saturation


def _thresholds(a):
    # an independent formulation: count the midpoints below a (ties to even)
    a = np.asarray(a, np.float64)
    return ((a > 0.25).astype(int) + (a >= 0.75) + (a > 1.25) + (a >= 1.75) + (a > 2.5) + (a >= 3.5)
            + (a > 5.0)).astype(np.uint8)


def test_nearest_value_by_midpoints():
    g = synth.rng(50)
    a = np.concatenate([g.random(20000) * 7.0, np.arange(0, 7, 0.125)])
    assert np.array_equal(mx.e2m1_round(a), _thresholds(a))


def test_block_exponent_rule():
    assert mx.block_exponent(np.float32(6.0)) == 0
    assert mx.block_exponent(np.float32(4.0)) == 0
    assert mx.block_exponent(np.float32(3.99)) == -1
    assert mx.block_exponent(np.float32(1.0)) == -2
    assert mx.block_exponent(np.float32(0.75)) == -3
    assert mx.block_exponent(np.float32(0.0)) == 0
    assert mx.block_exponent(np.float32(2.0 ** 127)) == 125
    assert mx.block_exponent(np.float32(2.0 ** 120)) == 118
    assert mx.block_exponent(np.float32(2.0 ** -140)) == -127  # clamped
    g = synth.rng(51)
    x = synth.laplace(g, (20, 64 * 32), 0.02)
    codes, e = mx.quantize_mxfp4(x)
    amax = np.abs(x.reshape(20, -1, 32)).max(axis=2)
    r = amax / np.ldexp(1.0, e)
    assert np.all((r >= 4) & (r < 8))  # the largest magnitude maps into [4, 8)


def test_representable_blocks_roundtrip():
    g = synth.rng(52)
    mags = mx.E2M1[g.integers(0, 8, size=(6, 128))]
    sign = np.where(g.random((6, 128)) < 0.5, -1.0, 1.0)
    v = mags * sign
    v[:, ::32] = 6.0  # every block's max is 6 -> e = 0
    ex = np.repeat(g.integers(-10, 10, size=(6, 4)), 32, axis=1)
    x = (v * np.ldexp(1.0, ex)).astype(np.float32)
    codes, e = mx.quantize_mxfp4(x)
    assert np.array_equal(mx.dequantize_mxfp4(codes, e), x.astype(np.float64))


def test_error_bound_and_signs():
    g = synth.rng(53)
    x = synth.gaussian(g, (16, 256), 1.0)
    x[0, :32] = 0.0
    x[1, 3] = -0.0
    codes, e = mx.quantize_mxfp4(x)
    assert np.all(codes[0, :32] == 0) and e[0, 0] == 0
    assert codes[1, 3] & 8 == 0
    X = np.repeat(np.ldexp(1.0, e), 32, axis=1)
    a = np.abs(x) / X
    err = np.abs(mx.dequantize_mxfp4(codes, e) - x) / X
    step = np.where(a < 2, 0.5, np.where(a < 4, 1.0, 2.0))
    sat = a > 6
    assert np.all(err[~sat] <= step[~sat] / 2 + 1e-12)
    assert np.all(err[sat] < 2.0)
    assert np.all(np.sign(mx.dequantize_mxfp4(codes, e)) * np.sign(x) >= 0)


def test_packing_layout_and_roundtrip():
    g = synth.rng(54)
    x = synth.gaussian(g, (3, 512), 1.0)
    codes, e = mx.quantize_mxfp4(x)
    packed, sc = mx.pack_mxfp4(codes, e)
    assert packed.shape == (3, 256) and sc.shape == (2, 3, 8)
    assert packed[1, 5] == codes[1, 10] | (codes[1, 11] << 4)  # low nibble = even element
    for r in range(3):
        for b in range(16):  # block b of row r: slice b // 8, position b % 8
            assert sc[b // 8, r, b % 8] == e[r, b] + 127
    c2, e2 = mx.unpack_mxfp4(packed, sc)
    assert np.array_equal(c2, codes) and np.array_equal(e2, e)


def test_product_against_exact_rationals():
    g = synth.rng(55)
    a = synth.gaussian(g, (2, 64), 1.0)
    b = synth.gaussian(g, (3, 64), 0.02)
    ca, ea = mx.quantize_mxfp4(a)
    cb, eb = mx.quantize_mxfp4(b)
    y = mx.gemm_mxfp4(ca, ea, cb, eb)

    def val(c, e, i, k):
        m = Fraction(float(mx.E2M1[c[i, k] & 7]))
        return (-m if c[i, k] & 8 else m) * Fraction(2) ** int(e[i, k // 32])
    for i in range(2):
        for j in range(3):
            exact = sum(val(ca, ea, i, k) * val(cb, eb, j, k) for k in range(64))
            assert y[i, j] == float(exact)
