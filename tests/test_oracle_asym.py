"""Pins of the oracle's asymmetric (zero-point) int8 quantization and of the
sign backbone + zero-point residual split and product.

Each pin comes from the pages or from mathematics, not from the oracle's own
formula: the range of [VG] fig. 22 with its ends on q_min / q_max and 0 on
the zero-point, the identity on integer data spanning the int8 range, brute
force over all 256 levels, power-of-two invariance, [OVR]'s division form of
the same quantizer, and exact rationals for the product."""
from fractions import Fraction

import numpy as np

import oracle
from oracle.numerics import bf16_bits_to_f32, f32_to_bf16_bits


def test_fig22_range_ends_and_zero():
    # [VG] fig. 22: the range [-7.59, 10.8]; the minimum goes to q_min, the
    # maximum to q_max, and 0 to the zero-point, which dequantizes to 0.
    # By hand: s = 255 / 18.39 = 13.866..., s * beta = -105.24...,
    # q_min - s * beta = -22.76 -> z = -23.
    x = np.array([[-7.59, 0.0, 10.8]], np.float32)
    q, s, z = oracle.quantize_asym(x)
    assert abs(float(s[0]) - 255 / 18.39) < 1e-5 * (255 / 18.39)
    assert int(z[0]) == -23
    assert q.tolist() == [[-128, -23, 127]]
    assert oracle.dequantize_asym(q, s[:, None], z[:, None])[0, 1] == 0.0


def test_integer_data_spanning_int8_is_identity():
    # data with min -128 and max 127: s = 255 / 255 = 1, z = -128 + 128 = 0, codes = data
    g = np.random.default_rng(11)
    x = g.integers(-128, 128, size=(6, 300)).astype(np.float32)
    x[:, 0], x[:, 1] = -128, 127
    q, s, z = oracle.quantize_asym(x)
    assert np.all(s == 1.0) and np.all(z == 0)
    assert np.array_equal(q.astype(np.float32), x)


def test_nearest_level_brute_force():
    # every code is the level (q - z) / s nearest to x, up to the fp32
    # rounding of s * x + z (far below half a level)
    g = np.random.default_rng(12)
    x = (g.standard_normal((5, 64)) * np.array([[0.1], [1.0], [3.0], [0.02], [7.0]]) +
         np.array([[0.0], [0.5], [-2.0], [0.01], [4.0]])).astype(np.float32)
    q, s, z = oracle.quantize_asym(x)
    levels = np.arange(-128, 128, dtype=np.float64)
    for r in range(x.shape[0]):
        grid = (levels - float(z[r])) / float(s[r])
        for c in range(x.shape[1]):
            d = np.abs(float(x[r, c]) - grid)
            got = d[int(q[r, c]) + 128]
            assert got <= d.min() + 1e-5 / float(s[r])
        assert np.all(np.diff(q[r][np.argsort(x[r], kind="stable")].astype(int)) >= 0)  # monotone


def test_power_of_two_scaling_keeps_codes():
    g = np.random.default_rng(13)
    x = (g.standard_normal((4, 128)) + 0.3).astype(np.float32)
    q0, s0, z0 = oracle.quantize_asym(x)
    for j in (-3, 5):
        q1, s1, z1 = oracle.quantize_asym((x * np.float32(2.0 ** j)).astype(np.float32))
        assert np.array_equal(q0, q1) and np.array_equal(z0, z1)
        assert np.array_equal(s1, (s0 / np.float32(2.0 ** j)).astype(np.float32))


def test_one_sided_and_zero_rows():
    x = np.array([[0.5, 1.0, 2.0, 4.0],       # positives only: beta widened to 0, z = q_min
                  [-4.0, -2.0, -1.0, -0.5],   # negatives only: alpha widened to 0, z = q_max
                  [0.0, 0.0, 0.0, 0.0]],      # all zero: s = 1, z = q_min, dequantized 0
                 np.float32)
    q, s, z = oracle.quantize_asym(x)
    assert z.tolist() == [-128, 127, -128]
    assert q[0, 3] == 127 and q[1, 0] == -128
    assert s[2] == 1.0 and np.all(q[2] == -128)
    assert np.all(oracle.dequantize_asym(q[2], s[2], z[2]) == 0.0)


def test_division_form_of_ovr_agrees():
    # [OVR] section 3 item 2 writes the same quantizer with the step
    # s' = (alpha - beta) / 255, z = round(-beta / s' + Q_min), q = round(x / s' + z).
    # It may differ from the multiplier form only where a value sits within
    # rounding of a half level: by at most 1, on a tiny fraction of values.
    g = np.random.default_rng(14)
    x = (g.standard_normal((64, 4096)) * 0.7 + 0.2).astype(np.float64)
    x32 = x.astype(np.float32)
    q, s, z = oracle.quantize_asym(x32)
    lo = np.minimum(x32.min(axis=1).astype(np.float64), 0.0)
    hi = np.maximum(x32.max(axis=1).astype(np.float64), 0.0)
    step = (hi - lo) / 255.0
    z2 = np.clip(np.rint(-lo / step - 128), -128, 127)
    q2 = np.clip(np.rint(x32 / step[:, None] + z2[:, None]), -128, 127)
    assert np.array_equal(z2.astype(np.int32), z)
    diff = np.abs(q2 - q)
    assert diff.max() <= 1 and np.count_nonzero(diff) <= 1e-4 * x.size


def test_zero_point_residual_reconstructs():
    g = np.random.default_rng(15)
    w = g.laplace(0.0, 0.015, size=(16, 512)).astype(np.float32)
    sign, alpha, rq, s_r, z_r = oracle.sign_residual_split_zp(w)
    sign0, alpha0, _, s_sym = oracle.sign_residual_split(w)
    assert np.array_equal(sign, sign0) and np.array_equal(alpha, alpha0)
    r = (w - (alpha[:, None] * sign.astype(np.float32)).astype(np.float32)).astype(np.float32)
    rhat = oracle.dequantize_asym(rq, s_r[:, None], z_r[:, None])
    err = np.abs(r.astype(np.float64) - rhat).max(axis=1)
    assert np.all(err <= 0.5 / s_r.astype(np.float64) * (1 + 1e-5))
    # 256 levels over [min, max] are never coarser than 255 over [-max|R|, max|R|]
    assert np.all(1.0 / s_r.astype(np.float64) <= 1.0 / s_sym.astype(np.float64) * (1 + 1e-6))
    assert np.all(rq.min(axis=1) == -128) and np.all(rq.max(axis=1) == 127)


def test_zero_point_product_exact_rationals():
    g = np.random.default_rng(16)
    n, k = 4, 4
    sign = np.where(g.random((n, k)) < 0.5, -1, 1).astype(np.int8)
    alpha = g.random(n).astype(np.float32)
    rq = g.integers(-128, 128, size=(n, k)).astype(np.int8)
    s_r = (g.random(n) * 100 + 1).astype(np.float32)
    z_r = g.integers(-128, 128, size=n).astype(np.int32)
    xb = f32_to_bf16_bits(g.standard_normal(k).astype(np.float32))
    x = bf16_bits_to_f32(xb)
    y = oracle.y_sign_residual_zp(sign, alpha, rq, s_r, z_r, xb)
    for i in range(n):
        xs = [Fraction(float(v)) for v in x]
        b = sum(int(sign[i, j]) * xs[j] for j in range(k))
        r = sum((int(rq[i, j]) - int(z_r[i])) * xs[j] for j in range(k))
        exact = Fraction(float(alpha[i])) * b + r / Fraction(float(s_r[i]))
        assert abs(Fraction(float(y[i])) - exact) <= abs(exact) * Fraction(1, 10 ** 12) + Fraction(1, 10 ** 15)
