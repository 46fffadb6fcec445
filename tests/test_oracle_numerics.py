"""Pins for the oracle's number-format helpers (CPU only).

Each check compares against something other than the helper itself: exact
rational arithmetic (fractions.Fraction), neighbouring fp32 values from
numpy.nextafter, math.fsum, or hand-computed bit patterns."""
import math
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.numerics import exact_abs_sum_units


def _nearest_f32_bruteforce(fr: Fraction) -> np.float32:
    """Nearest fp32 to a positive rational, found by testing neighbours."""
    c = np.float32(float(fr))  # within one or two ulps of the answer
    cands = {c}
    for _ in range(3):
        cands |= {np.nextafter(v, np.float32(np.inf)) for v in cands}
        cands |= {np.nextafter(v, np.float32(0)) for v in cands}
    cands = sorted(v for v in cands if np.isfinite(v))
    best = min(cands, key=lambda v: (abs(Fraction(float(v)) - fr),
                                     int(np.array(v, np.float32).view(np.uint32)) & 1))
    return best


@pytest.mark.parametrize("seed", range(6))
def test_round_rational_matches_bruteforce(seed):
    g = np.random.default_rng(seed)
    for _ in range(300):
        num = int(g.integers(1, 2 ** 62)) >> int(g.integers(0, 60))
        den = int(g.integers(1, 2 ** 62)) >> int(g.integers(0, 60))
        scale = int(g.integers(-150, 120))
        if scale >= 0:
            num <<= scale
        else:
            den <<= -scale
        num = max(num, 1)
        den = max(den, 1)
        fr = Fraction(num, den)
        if fr > Fraction(float(np.finfo(np.float32).max)):
            continue
        got = oracle.round_rational_to_f32(num, den)
        want = _nearest_f32_bruteforce(fr)
        assert got == want, (num, den, got, want)


def test_round_rational_ties_and_exact():
    # exactly representable values come back unchanged
    for v in [1.0, 0.5, 3.0, 2.0 ** -149, 2.0 ** -126, 1.5 * 2.0 ** 100]:
        fr = Fraction(v)
        assert oracle.round_rational_to_f32(fr.numerator, fr.denominator) == np.float32(v)
    # 1 + 2^-24 is halfway between 1 and 1 + 2^-23: ties to even -> 1
    assert oracle.round_rational_to_f32(2 ** 24 + 1, 2 ** 24) == np.float32(1.0)
    # 1 + 3*2^-24 is halfway between 1+2^-23 (odd) and 1+2^-22 (even) -> up
    assert oracle.round_rational_to_f32(2 ** 24 + 3, 2 ** 24) == np.float32(1 + 2 ** -22)
    # halfway below the smallest subnormal: ties to even (0)
    assert oracle.round_rational_to_f32(1, 2 ** 150) == np.float32(0.0)
    assert oracle.round_rational_to_f32(3, 2 ** 150) == np.float32(2.0 ** -148)
    # 127 / 10.8 in fp32 equals IEEE division of the fp32 operands
    a = Fraction(float(np.float32(10.8)))
    q = Fraction(127) / a
    assert oracle.round_rational_to_f32(q.numerator, q.denominator) == np.float32(127) / np.float32(10.8)


def test_bf16_conversions():
    bits = oracle.f32_to_bf16_bits(np.array([1.0, -2.0, 1 + 2 ** -8, 1 + 3 * 2 ** -8, 1 + 2 ** -7,
                                             1 + 2 ** -8 + 2 ** -20, 0.0, -0.0], np.float32))
    # 1.0 = 0x3F80; -2 = 0xC000; tie at 1+2^-8 -> even (0x3F80); 1+3*2^-8 tie -> 0x3F82;
    # 1+2^-7 exact 0x3F81; just above the tie rounds up 0x3F81
    assert bits.tolist() == [0x3F80, 0xC000, 0x3F80, 0x3F82, 0x3F81, 0x3F81, 0x0000, 0x8000]
    back = oracle.bf16_bits_to_f32(bits)
    assert back[0] == 1.0 and back[1] == -2.0 and back[3] == np.float32(1 + 2 ** -6)
    g = np.random.default_rng(0)
    x = g.standard_normal(10000).astype(np.float32)
    b = oracle.f32_to_bf16_bits(x)
    y = oracle.bf16_bits_to_f32(b)
    # nearest: |x - y| <= half a bf16 ulp, and y is bf16-representable
    ulp = np.ldexp(np.float64(1), (np.frexp(y.astype(np.float64))[1] - 8).astype(np.int64))
    assert np.all(np.abs(x.astype(np.float64) - y) <= ulp / 2 + 1e-30)
    assert np.all((y.view(np.uint32) & 0xFFFF) == 0)


def _fraction_abs_sum(a):
    return sum((Fraction(float(v)) for v in np.abs(a.astype(np.float64)).ravel()), Fraction(0))


@pytest.mark.parametrize("seed", range(5))
def test_exact_abs_sum_units(seed):
    g = np.random.default_rng(seed)
    a = (g.standard_normal(500) * np.exp(g.uniform(-100, 80, 500))).astype(np.float32)
    a[:5] = [0.0, -0.0, np.float32(2.0 ** -149), np.float32(-(2.0 ** -130)), np.finfo(np.float32).max / 1000]
    s = exact_abs_sum_units(a)
    assert Fraction(s, 2 ** 149) == _fraction_abs_sum(a)


@pytest.mark.parametrize("seed", range(5))
def test_mean_abs_matches_fraction_and_fsum(seed):
    g = np.random.default_rng(100 + seed)
    a = g.laplace(0, 0.02, size=(37, 29)).astype(np.float32)
    a[0, :3] = [0.0, -0.0, 1e-40]
    exact = _fraction_abs_sum(a) / a.size
    want = _nearest_f32_bruteforce(exact)
    got = oracle.mean_abs_f32(a)
    assert got == want
    fs = np.float32(math.fsum(np.abs(a.astype(np.float64)).ravel()) / a.size)
    assert abs(int(got.view(np.int32)) - int(np.array(fs).view(np.int32))) <= 1
    rows = oracle.mean_abs_rows_f32(a)
    assert all(rows[i] == oracle.mean_abs_f32(a[i]) for i in range(a.shape[0]))


def test_mean_abs_special_cases():
    # constant magnitude c: the mean is exactly c
    for c in [0.02, 3.0, 1e-38, 2.0 ** -149]:
        a = np.array([c, -c, c, -c, c], np.float32)
        assert oracle.mean_abs_f32(a) == np.float32(c)
    assert oracle.mean_abs_f32(np.zeros(7, np.float32)) == 0
    # the mean of [1, 2] is 1.5, of [1, 2, 2] is 5/3 rounded
    assert oracle.mean_abs_f32(np.array([1, -2], np.float32)) == np.float32(1.5)
    assert oracle.mean_abs_f32(np.array([1, 2, 2], np.float32)) == np.float32(5.0 / 3.0)


def _pyint_abs_sum_units(a) -> int:
    """sum |a_i| * 2**149 with Python integers, element by element: every
    fp32 value times 2**149 is an integer, exact in fp64 (a power-of-two
    scaling) and converted exactly by int().  No binade decomposition."""
    flat = np.abs(np.ascontiguousarray(a, np.float32).ravel()).astype(np.float64) * 2.0 ** 149
    total = 0
    for lo in range(0, flat.size, 1 << 20):
        total += sum(map(int, flat[lo:lo + (1 << 20)].tolist()))
    return total


def test_mean_abs_at_ternary_workload_size():
    # gamma of the ternary decode workload (11008 x 4096 = 45,088,768
    # Laplace weights, [VG] 'BitNet b1.58' Fig. 60): the oracle's binade sums
    # against a plain integer sum, and its rounding against a search of the
    # neighbouring fp32 values
    import synth
    w = synth.ternary_decode().tensors["w"]
    s = _pyint_abs_sum_units(w)
    assert exact_abs_sum_units(w) == s
    assert oracle.mean_abs_f32(w) == _nearest_f32_bruteforce(Fraction(s, w.size << 149))


def test_mean_abs_rows_at_separated_workload_shape():
    # per-row alpha of the separated decode workload (rows of 8192 Laplace
    # weights with 0.5% x20 outliers, [SEP] section 2.1), on a sample of rows
    import synth
    rows = np.random.default_rng(5).choice(28672, 96, replace=False)
    w = synth.sign_residual_decode(rows=np.sort(rows)).tensors["w"]
    got = oracle.mean_abs_rows_f32(w)
    for i in range(w.shape[0]):
        s = _pyint_abs_sum_units(w[i])
        assert got[i] == _nearest_f32_bruteforce(Fraction(s, w.shape[1] << 149))
