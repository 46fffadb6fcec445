"""Pins for the oracle's quantizers (CPU only)."""
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


def _rne(fr: Fraction) -> int:
    fl = fr.numerator // fr.denominator
    rem = fr - fl
    if rem > Fraction(1, 2) or (rem == Fraction(1, 2) and fl % 2):
        fl += 1
    return fl


def _code_exact(x: np.float32, s: np.float32) -> int:
    """clip(rne(fl32(x * s))) with the fp32 product rounded by exact rationals."""
    p = Fraction(float(x)) * Fraction(float(s))
    mag = abs(p)
    t = oracle.round_rational_to_f32(mag.numerator, mag.denominator) if mag else np.float32(0)
    t = Fraction(float(t)) * (1 if p >= 0 else -1)
    return max(-127, min(127, _rne(t)))


# ---------------------------------------------------------------- absmax

def test_worked_example():
    g = _golden("absmax_worked_example.json")
    x = np.array(g["values"], np.float32)
    q, s = oracle.quantize_absmax(x, per_row=False)
    assert np.float32(np.max(np.abs(x))) == np.float32(g["alpha"])
    assert q[1] == g["printed"]["code_of_3.08"] and q[2] == g["printed"]["code_of_3.02"]
    assert q[0] == g["derived"]["code_of_10.8"] and q[3] == g["derived"]["code_of_-7.59"]
    assert abs(float(oracle.dequantize(36, s[0])) - g["printed"]["dequantized_36_2dp"]) < 0.005
    # the scale is the multiplier q_max / alpha, rounded once to fp32
    a = Fraction(float(np.float32(g["alpha"])))
    r = Fraction(127) / a
    assert s[0] == oracle.round_rational_to_f32(r.numerator, r.denominator)
    assert abs(float(s[0]) - 127 / 10.8) < 1e-5


@pytest.mark.parametrize("seed", range(4))
def test_absmax_codes_match_exact_rationals(seed):
    g = np.random.default_rng(seed)
    x = (g.standard_normal((6, 40)) * np.exp(g.uniform(-20, 20, (6, 1)))).astype(np.float32)
    q, s = oracle.quantize_absmax(x, per_row=True)
    for r in range(x.shape[0]):
        alpha = Fraction(float(np.max(np.abs(x[r]))))
        sr = Fraction(127) / alpha
        assert s[r] == oracle.round_rational_to_f32(sr.numerator, sr.denominator)
        for c in range(x.shape[1]):
            assert q[r, c] == _code_exact(x[r, c], s[r])


def test_absmax_near_ties_are_half_even():
    # values whose scaled product lands exactly on .5 in fp32
    x = np.array([127.0, 0.5, 1.5, 2.5, -0.5, -2.5, 3.0], np.float32)
    q, s = oracle.quantize_absmax(x, per_row=False)
    assert s[0] == 1.0
    assert q.tolist() == [127, 0, 2, 2, 0, -2, 3]


@pytest.mark.parametrize("seed", range(4))
def test_absmax_invariants(seed):
    g = np.random.default_rng(10 + seed)
    x = (g.standard_normal((16, 257)) * 0.02).astype(np.float32)
    q, s = oracle.quantize_absmax(x, per_row=True)
    assert q.dtype == np.int8 and np.all(np.abs(q.astype(int)) <= 127) and not np.any(q == -128)
    am = np.argmax(np.abs(x), axis=1)
    assert np.all(np.abs(q[np.arange(16), am].astype(int)) == 127)
    qn, sn = oracle.quantize_absmax(-x, per_row=True)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for j in (-3, 5):
        qj, sj = oracle.quantize_absmax((x * np.float32(2.0 ** j)).astype(np.float32), per_row=True)
        assert np.array_equal(qj, q)
    # round-trip error within half a step ([VG] Fig. 21 quantization error)
    err = np.abs(x.astype(np.float64) - oracle.dequantize(q, s[:, None]))
    assert np.all(err <= 0.5 / s[:, None].astype(np.float64) * (1 + 1e-6))
    # re-quantizing the dequantized value gives the same code
    xd = (q.astype(np.float32) / s[:, None]).astype(np.float32)
    assert np.array_equal(oracle.quantize_with_scale(xd, s[:, None]), q)


def test_absmax_granularity_and_zero_group():
    g = np.random.default_rng(3)
    x = g.standard_normal((5, 64)).astype(np.float32)
    x[2] = 0
    q, s = oracle.quantize_absmax(x, per_row=True)
    assert s[2] == 1 and not q[2].any()
    for r in (0, 1, 3):
        q1, s1 = oracle.quantize_absmax(x[r], per_row=False)
        assert np.array_equal(q1, q[r]) and s1[0] == s[r]
    qt, st = oracle.quantize_absmax(x, per_row=False)
    assert st[0] == np.float32(127) / np.max(np.abs(x))
    assert oracle.quantize_absmax(np.zeros(9, np.float32), per_row=False)[1][0] == 1



def test_absmax_scale_clamped_for_tiny_groups():
    # 127 / alpha overflows fp32 for alpha below 127 / FLT_MAX: the scale is
    # clamped to FLT_MAX (reading of the pages' s = q_max / alpha, [VG]
    # 'Symmetric quantization', for a range the fp32 quotient cannot hold)
    fmax = np.finfo(np.float32).max
    x = np.array([1e-37, -5e-38, 0.0, -0.0, 3e-38, 2.0 ** -149, 3.5e-37, -1e-38], np.float32)
    q, s = oracle.quantize_absmax(x, per_row=False)
    assert s[0] == fmax and np.isfinite(s).all()
    # fl32(x * s): the fp64 product of two fp32 values is exact, so one
    # narrowing to fp32 rounds it once; then half-even rounding and the clip
    t = (x.astype(np.float64) * np.float64(fmax)).astype(np.float32)
    assert np.array_equal(q, np.clip(np.rint(t), -127, 127).astype(np.int8))
    assert q[2] == 0 and q[3] == 0 and q[0] == 34 and q[6] == 119
    assert np.array_equal(oracle.quantize_absmax(-x, per_row=False)[0], -q)
    # per row: only the tiny row is clamped; a row just above the bound is not
    rows = np.stack([x, x * np.float32(1e30), np.full(8, 127 / fmax * 1.01, np.float32)])
    qr, sr = oracle.quantize_absmax(rows, per_row=True)
    assert sr[0] == fmax and sr[1] == np.float32(127) / np.max(np.abs(rows[1])) and sr[2] < fmax
    assert np.array_equal(qr[0], q) and (qr[2] == 127).all()
    # asymmetric: 255 / d overflows likewise (d = 3e-38); 0 still maps to z
    lo, hi = np.float32(-1e-38), np.float32(2e-38)
    sa, za = oracle.asym_params(np.array([lo]), np.array([hi]))
    assert sa[0] == fmax
    zt = np.float32(-128) - (np.float64(fmax) * np.float64(lo)).astype(np.float32)
    assert za[0] == np.rint(zt) == -125
    xa = np.array([lo, 0.0, hi], np.float32)
    qa = oracle.quantize_with_zero_point(xa, sa, za)
    ta = ((xa.astype(np.float64) * np.float64(fmax)).astype(np.float32) + np.float32(za[0])).astype(np.float32)
    assert np.array_equal(qa, np.clip(np.rint(ta), -128, 127).astype(np.int8)) and qa[1] == za[0]


# ---------------------------------------------------------------- ternary

def test_ternary_codes_and_scale():
    w = synth.ternary_decode(n=64, k=256, seed=3).tensors["w"]
    q, gamma = oracle.ternary_absmean(w)
    assert set(np.unique(q).tolist()) <= {-1, 0, 1}
    exact = sum((Fraction(float(v)) for v in np.abs(w.astype(np.float64)).ravel()), Fraction(0)) / w.size
    assert gamma == oracle.round_rational_to_f32(exact.numerator, exact.denominator)
    small = np.abs(w) < 0.49 * gamma
    assert not q[small].any()
    big = np.abs(w) > 1.51 * gamma
    assert np.array_equal(q[big], np.sign(w[big]).astype(np.int8))


def test_ternary_special_cases():
    # weights already in {-c, 0, c}: codes are the sign pattern exactly
    g = np.random.default_rng(1)
    c = np.float32(0.037)
    pat = g.integers(-1, 2, size=(8, 32))
    q, gamma = oracle.ternary_absmean((pat * c).astype(np.float32))
    assert np.array_equal(q, pat.astype(np.int8))
    # exact halves round to even: W/gamma = 0.5 -> 0, 1.5 -> 2 -> clipped to 1
    q, gamma = oracle.ternary_absmean(np.array([0.5, 1.5, 1.0, -1.0], np.float32))
    assert gamma == 1.0 and q.tolist() == [0, 1, 1, -1]
    q, gamma = oracle.ternary_absmean(np.zeros((3, 4), np.float32))
    assert gamma == 0 and not q.any()


def test_ternary_dot_example():
    g = _golden("small_examples.json")["ternary_dot"]
    w = np.array([g["weights"]], np.int8)
    x = np.array([5, -7, 11, 13], np.int8)
    want = int(x[0]) - int(x[1]) - int(x[2]) + int(x[3])
    assert oracle.int_dot_bruteforce(w, x)[0] == want
    assert oracle.int_dot_exact(w, x)[0] == want


# ---------------------------------------------------------------- sign + residual

def test_sign_residual_definitions():
    wl = synth.sign_residual_decode(n=24, k=512, seed=4).tensors["w"]
    w = wl.copy()
    w[0, :4] = [0.0, -0.0, 1e-8, -1e-8]
    sign, alpha, rq, s_r = oracle.sign_residual_split(w)
    assert sign[0, 0] == 1 and sign[0, 1] == 1 and sign[0, 2] == 1 and sign[0, 3] == -1
    assert set(np.unique(sign).tolist()) <= {-1, 1}
    for r in range(w.shape[0]):
        ex = sum((Fraction(float(v)) for v in np.abs(w[r].astype(np.float64))), Fraction(0)) / w.shape[1]
        assert alpha[r] == oracle.round_rational_to_f32(ex.numerator, ex.denominator)
    # alpha minimises ||W - a sign(W)||^2 (closed form: mean |W|)
    w64 = w.astype(np.float64)
    for r in range(4):
        def loss(a):
            return float(np.sum((w64[r] - a * sign[r]) ** 2))
        a0 = float(alpha[r])
        assert loss(a0) <= loss(a0 * (1 + 1e-3)) and loss(a0) <= loss(a0 * (1 - 1e-3))
    # backbone + unquantized residual gives back W to within half an ulp of R
    r_f32 = (w - (alpha[:, None] * sign).astype(np.float32)).astype(np.float32)
    recon = alpha[:, None].astype(np.float64) * sign + r_f32.astype(np.float64)
    ulp = np.spacing(np.abs(r_f32)).astype(np.float64)
    assert np.all(np.abs(recon - w64) <= ulp / 2)
    # the residual's int8 codes are the per-row absmax codes of R with its own scale
    q_ref, s_ref = oracle.quantize_absmax(r_f32, per_row=True)
    assert np.array_equal(q_ref, rq) and np.array_equal(s_ref, s_r)
    err = np.abs(r_f32.astype(np.float64) - oracle.dequantize(rq, s_r[:, None]))
    assert np.all(err <= 0.5 / s_r[:, None].astype(np.float64) * (1 + 1e-6))


def test_residual_recovers_what_the_backbone_drops():
    wl = synth.sign_residual_decode(n=64, k=1024, seed=4)
    w = wl.tensors["w"]
    xb = wl.tensors["x_bf16"]
    x = oracle.bf16_bits_to_f32(xb)
    sign, alpha, rq, s_r = oracle.sign_residual_split(w)
    y_sep = oracle.y_sign_residual(sign, alpha, rq, s_r, xb)
    y_sign_only = oracle.y_sign_residual(sign, alpha, np.zeros_like(rq), np.ones_like(s_r), xb)
    e_sep = oracle.relative_method_error(y_sep, w, x)
    e_sign = oracle.relative_method_error(y_sign_only, w, x)
    assert e_sep < 0.05 < e_sign


def test_all_zero_row_split():
    w = np.zeros((2, 16), np.float32)
    w[1] = np.linspace(-1, 1, 16, dtype=np.float32)
    sign, alpha, rq, s_r = oracle.sign_residual_split(w)
    assert alpha[0] == 0 and s_r[0] == 1 and not rq[0].any() and np.all(sign[0] == 1)


# ---------------------------------------------------------------- outlier split

def test_outlier_split():
    wl = synth.prefill_outlier(m=32, k=512, n=64, n_out=6, seed=5)
    xb, idx = wl.tensors["x_bf16"], wl.tensors["idx"]
    xq, s, xo = oracle.outlier_split_quantize(xb, idx)
    x = oracle.bf16_bits_to_f32(xb)
    keep = np.ones(512, bool)
    keep[idx] = False
    assert np.array_equal(xo, xb[:, idx])
    assert not xq[:, idx].any()
    q_ref, s_ref = oracle.quantize_absmax(x[:, keep], per_row=True)
    assert np.array_equal(s, s_ref) and np.array_equal(xq[:, keep], q_ref)
    # the outlier channels really are ~50x larger
    assert np.median(np.abs(x[:, idx])) > 20 * np.median(np.abs(x[:, keep]))
    # no outliers: plain per-token absmax
    q0, s0, xo0 = oracle.outlier_split_quantize(xb, np.zeros(0, np.int32))
    q_ref, s_ref = oracle.quantize_absmax(x, per_row=True)
    assert np.array_equal(q0, q_ref) and np.array_equal(s0, s_ref) and xo0.shape == (32, 0)
    # every channel an outlier: nothing left for int8
    qa, sa, _ = oracle.outlier_split_quantize(xb[:, :8], np.arange(8, dtype=np.int32))
    assert not qa.any() and np.all(sa == 1)


def test_gather_outlier_weights():
    w = np.array([[1.0, 1 + 2 ** -8, 3.0], [1 + 3 * 2 ** -8, -2.0, 0.5]], np.float32)
    got = oracle.gather_outlier_weights(w, np.array([1, 0], np.int32))
    assert got.tolist() == [[0x3F80, 0x3F80], [0xC000, 0x3F82]]


def test_ternary_divides_rather_than_multiplying_by_reciprocal():
    # W = [w, y] with exact mean gamma = (w + y) / 2 and w / gamma just above
    # 0.5: fl32(w / gamma) rounds up to code 1, while w * fl32(1 / gamma)
    # lands on 0.5 and rounds (half-even) to 0.  The definition divides.
    w = np.array([1.9486494, 5.8459477], np.float32)
    q, gamma = oracle.ternary_absmean(w)
    assert float(gamma) == (float(w[0]) + float(w[1])) / 2
    assert q.tolist() == [1, 1]
    recip = np.clip(np.rint((w * (np.float32(1) / gamma)).astype(np.float32)), -1, 1)
    assert recip.tolist() == [0, 1]


def test_detect_outlier_channels():
    bf = synth.to_bf16_bits
    # hand-worked: channel ranges (max |x| over rows) are 1, 5, 7, 5
    x = bf(np.array([[1.0, -5.0, 2.0, 5.0], [0.0, 3.0, -7.0, 1.0]], np.float32))
    assert oracle.detect_outlier_channels(x, 1).tolist() == [2]
    assert oracle.detect_outlier_channels(x, 2).tolist() == [1, 2]      # tie 5 = 5 goes to the lower index
    assert oracle.detect_outlier_channels(x, 3).tolist() == [1, 2, 3]
    assert oracle.detect_outlier_channels(x, 4).tolist() == [0, 1, 2, 3]
    assert oracle.detect_outlier_channels(x, 0).tolist() == []
    # all ranges equal: the lowest channels
    z = np.zeros((3, 16), np.uint16)
    assert oracle.detect_outlier_channels(z, 5).tolist() == [0, 1, 2, 3, 4]
    # the channels the generator scales x50 stand out by far and are found exactly
    for (m, k, n_out, seed) in [(64, 256, 4, 5), (512, 4096, 20, 5), (8, 1024, 12, 9)]:
        wl = synth.prefill_outlier(m=m, k=k, n=8, n_out=n_out, seed=seed)
        got = oracle.detect_outlier_channels(wl.tensors["x_bf16"], n_out)
        assert got.tolist() == wl.tensors["idx"].tolist()
        assert got.dtype == np.int32
