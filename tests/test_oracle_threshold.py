"""Pins of the thresholded separated-quantization oracle ([SEP] sections
2.1, 3.2, 3.3, 5.2, 5.3) against library routines, closed forms, brute
force and the special cases that reduce to other quantizers."""
from fractions import Fraction

import numpy as np
import pytest

import oracle
import oracle.threshold as th
import synth


def test_nearest_rank_is_numpys_inverted_cdf_percentile():
    g = synth.rng(30)
    for k in (7, 64, 100, 1152, 4096):
        a = np.abs(synth.laplace(g, (k,), 1.0)).astype(np.float32)
        for p in (1, 30, 50, 70, 80, 99, 100):
            tau, _ = th.row_thresholds(a, p, 0)
            ref = np.percentile(a.astype(np.float64), p, method="inverted_cdf")
            assert tau == np.float32(ref), (k, p)
            # the defining property: the smallest magnitude that at least p% of the row does not exceed
            assert np.sum(a <= tau) * 100 >= p * k
            assert np.sum(a < tau) * 100 < p * k


def test_class_shares_match_the_pages_figures():
    # distinct magnitudes: |B| = K - j(80), |Z| = j(50), |R| = the rest
    k = 4096
    w = synth.gaussian(synth.rng(31), (3, k), 0.02)
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 50)
    for r in range(3):
        nb = int(np.sum((fields[r] == 0) | (fields[r] == 2)))
        nz = int(np.sum(fields[r] == 1))
        nr = int(np.sum(fields[r] == 3))
        assert nb == k - th.nearest_rank(80, k) and nz == th.nearest_rank(50, k) and nb + nz + nr == k
        # section 3.2: the residual holds about 30% of the weights;
        # section 3.3: the residual matrix (all but the backbone) is 50-70% zero
        assert abs(nr / k - 0.30) < 1e-3
        sparsity = nz / (nz + nr)
        assert 0.5 <= sparsity <= 0.7
    plane, stream = th.pack_threshold(fields, rq, th.resid_ld(k, 50))
    assert plane.nbytes == 3 * k // 4  # 2 bits per weight for the classes


def test_classes_follow_the_thresholds():
    g = synth.rng(32)
    w = synth.laplace(g, (5, 640), 0.015)
    synth.boost_entries(g, w, 0.005, 20.0)
    for pb, pz in ((80, 50), (70, 40), (90, 0), (60, 60)):
        fields, alpha, rq, s_r = th.threshold_split(w, pb, pz)
        for r in range(5):
            row = w[r]
            mag = np.abs(row)
            srt = np.sort(mag)
            tau = srt[(pb * 640 + 99) // 100 - 1]
            b = mag > tau
            assert np.array_equal(fields[r] == 2, b & (row > 0))
            assert np.array_equal(fields[r] == 0, b & (row < 0))
            if pz:
                eps = srt[(pz * 640 + 99) // 100 - 1]
                assert np.array_equal(fields[r] == 1, mag <= eps)
            else:
                assert not np.any(fields[r] == 1)  # no zero class
            # residual codes only on R, and within half a step of the weight
            res = fields[r] == 3
            assert not np.any(rq[r][~res])
            if res.any():
                err = np.abs(rq[r][res] / np.float64(s_r[r]) - row[res])
                assert np.all(err <= 0.5 / np.float64(s_r[r]) * (1 + 1e-6))
                assert np.max(np.abs(rq[r][res])) == 127  # the largest residual magnitude maps to 127


def test_alpha_is_the_least_squares_backbone_scale():
    w = synth.laplace(synth.rng(33), (4, 1024), 0.02)
    fields, alpha, rq, s_r = th.threshold_split(w, 75, 25)
    for r in range(4):
        b = (fields[r] == 0) | (fields[r] == 2)
        mag = np.abs(w[r][b]).astype(np.float64)

        def err(a):
            return float(np.sum((mag - np.float64(a)) ** 2))

        a = alpha[r]
        up = np.nextafter(a, np.float32(np.inf))
        dn = np.nextafter(a, np.float32(0))
        assert err(a) <= err(up) and err(a) <= err(dn)  # the best fp32 backbone scale
        # and it is the correctly rounded mean
        exact = sum(Fraction(float(v)) for v in mag) / int(b.sum())
        assert abs(Fraction(float(a)) - exact) <= Fraction(float(np.spacing(a))) / 2


def test_no_backbone_reduces_to_per_row_absmax():
    # pct_backbone = 100, pct_zero = 0: tau = max|w|, B and Z empty, R = all
    w = synth.gaussian(synth.rng(34), (6, 512), 0.02)
    fields, alpha, rq, s_r = th.threshold_split(w, 100, 0)
    q_ref, s_ref = oracle.quantize_absmax(w, per_row=True)
    assert np.all(fields == 3) and not alpha.any()
    assert np.array_equal(rq, q_ref) and np.array_equal(s_r, s_ref)


def test_no_residual_is_a_thresholded_sign():
    # pct_zero = pct_backbone: R is empty, the weights are +-alpha or 0
    w = synth.laplace(synth.rng(35), (3, 256), 0.02)
    fields, alpha, rq, s_r = th.threshold_split(w, 70, 70)
    for r in range(3):
        tau = np.sort(np.abs(w[r]))[(70 * 256 + 99) // 100 - 1]
        ref = np.where(np.abs(w[r]) > tau, np.sign(w[r]), 0).astype(np.int64) + 1
        assert np.array_equal(fields[r].astype(np.int64), ref)
    assert not rq.any() and np.all(s_r == 1)


def test_equal_magnitudes_and_zero_rows():
    w = np.zeros((3, 128), np.float32)
    w[1, :] = 0.5
    w[2, ::2] = -0.25
    w[2, 1::2] = 0.25
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 50)
    # every magnitude equals both thresholds: nothing is above tau, all is <= eps
    assert np.all(fields == 1) and not alpha.any() and not rq.any() and np.all(s_r == 1)
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 0)
    assert np.all(fields == 3) and not alpha.any()
    assert np.all(rq[1] == 127) and np.array_equal(rq[2], np.where(w[2] > 0, 127, -127))
    assert s_r[0] == 1 and not rq[0].any()


def _pack_loops(fields, rq, ld):
    n, k = fields.shape
    plane = np.zeros((n, k // 4), np.uint8)
    stream = np.zeros((n, ld), np.int8)
    for r in range(n):
        j = 0
        for c in range(k):
            plane[r, c // 4] |= int(fields[r, c]) << (2 * (c % 4))
            if fields[r, c] == 3:
                stream[r, j] = rq[r, c]
                j += 1
    return plane, stream


def test_packing_layout_and_roundtrip():
    w = synth.laplace(synth.rng(36), (4, 384), 0.02)
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 30)
    ld = th.resid_ld(384, 30)
    assert ld % 16 == 0 and ld >= 384 - th.nearest_rank(30, 384)
    plane, stream = th.pack_threshold(fields, rq, ld)
    p2, s2 = _pack_loops(fields, rq, ld)
    assert np.array_equal(plane, p2) and np.array_equal(stream, s2)
    f3, rq3 = th.unpack_threshold(plane, stream, 384)
    assert np.array_equal(f3, fields) and np.array_equal(rq3, rq)
    with pytest.raises(ValueError):
        th.pack_threshold(fields, rq, 16)


def test_products_against_exact_rationals():
    g = synth.rng(37)
    w = synth.laplace(g, (3, 64), 0.02)
    x = synth.gaussian(g, (64,), 1.0)
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 50)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    acc_b, acc_r = th.int_products(fields, rq, xq)
    for r in range(3):
        ab = sum((1 if fields[r, c] == 2 else -1 if fields[r, c] == 0 else 0) * int(xq[c]) for c in range(64))
        ar = sum(int(rq[r, c]) * int(xq[c]) for c in range(64))
        assert acc_b[r] == ab and acc_r[r] == ar
    y = th.y_threshold(acc_b, acc_r, alpha, s_r, s_x)
    sx = Fraction(float(s_x[0]))
    for r in range(3):
        a, sr = Fraction(float(alpha[r])), Fraction(float(s_r[r]))
        wv = [a if fields[r, c] == 2 else -a if fields[r, c] == 0 else Fraction(int(rq[r, c])) / sr
              for c in range(64)]
        exact = sum(wv[c] * int(xq[c]) for c in range(64)) / sx
        assert abs(y[r] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    yb = th.y_threshold(acc_b, acc_r, alpha, s_r, s_x, skip_residual=True)
    assert np.allclose(yb, alpha.astype(np.float64) * acc_b / np.float64(s_x[0]), rtol=0, atol=0)


def test_threshold_backbone_beats_dense_sign_only():
    # method error (reported): the split approximates W better than alpha * sign(W)
    w = synth.laplace(synth.rng(38), (8, 2048), 0.015)
    fields, alpha, rq, s_r = th.threshold_split(w, 80, 50)
    what = th.dequantize_threshold(fields, alpha, rq, s_r)
    sign, a_dense, _, _ = oracle.sign_residual_split(w)
    sign_only = a_dense[:, None].astype(np.float64) * sign
    e_split = np.linalg.norm(what - w) / np.linalg.norm(w)
    e_sign = np.linalg.norm(sign_only - w) / np.linalg.norm(w)
    assert e_split < e_sign
