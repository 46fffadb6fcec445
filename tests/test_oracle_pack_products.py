"""Pins for the oracle's packing and product references (CPU only)."""
import itertools
import json
import os
from fractions import Fraction

import numpy as np
import pytest

import oracle
from oracle.products import _check_exact
import synth

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden(name):
    with open(os.path.join(GOLDEN, name)) as f:
        return json.load(f)


# ---------------------------------------------------------------- packing

def test_ternary_pack_exhaustive():
    tuples = np.array(list(itertools.product([-1, 0, 1], repeat=4)), np.int8)  # 81 rows of 4
    p = oracle.pack(tuples, 2)
    assert p.shape == (81, 1)
    assert np.array_equal(p, oracle.pack_loops(tuples, 2))
    assert len(set(p.ravel().tolist())) == 81
    assert np.array_equal(oracle.unpack(p, 2, 4), tuples)
    assert np.array_equal(oracle.unpack_loops(p, 2, 4), tuples)
    # hand-worked byte: codes [-1, 0, 1, 1] -> fields [0, 1, 2, 2] -> 0 + 4 + 32 + 128
    assert oracle.pack(np.array([[-1, 0, 1, 1]], np.int8), 2)[0, 0] == 164


def test_sign_pack_exhaustive():
    allbytes = np.arange(256, dtype=np.uint8)[:, None]
    codes = oracle.unpack(allbytes, 1, 8)
    assert np.array_equal(codes, oracle.unpack_loops(allbytes, 1, 8))
    assert np.array_equal(oracle.pack(codes, 1), allbytes)
    assert np.array_equal(oracle.pack_loops(codes, 1), allbytes)
    # byte 0b00000101: codes +1 at positions 0 and 2
    assert codes[5].tolist() == [1, -1, 1, -1, -1, -1, -1, -1]


@pytest.mark.parametrize("bits", [1, 2])
def test_pack_random_shapes(bits):
    g = np.random.default_rng(bits)
    for n, k in [(1, 8), (3, 24), (7, 128), (5, 40)]:
        if bits == 2:
            c = g.integers(-1, 2, size=(n, k)).astype(np.int8)
        else:
            c = np.where(g.random((n, k)) < 0.5, -1, 1).astype(np.int8)
        p = oracle.pack(c, bits)
        assert p.shape == (n, k * bits // 8) and p.dtype == np.uint8
        assert np.array_equal(p, oracle.pack_loops(c, bits))
        assert np.array_equal(oracle.unpack(p, bits, k), c)


def test_pack_rejects_bad_codes():
    with pytest.raises(ValueError):
        oracle.pack(np.array([[2, 0, 0, 0]], np.int8), 2)
    with pytest.raises(ValueError):
        oracle.pack(np.array([[0] * 8], np.int8), 1)
    with pytest.raises(ValueError):
        oracle.pack(np.zeros((1, 6), np.int8), 2)


def test_byte_accounting():
    g = _golden("small_examples.json")
    b = g["bytes_per_weight"]
    assert abs(b["sign_bytes"] * b["backbone_share"] + b["int8_bytes"] * b["residual_share"] - b["total"]) < 1e-12
    # packed sizes: one sign bit and two ternary bits per weight
    assert oracle.pack(np.ones((4, 64), np.int8), 1).nbytes * 8 == 4 * 64 * b["sign_bytes"] * 8
    assert oracle.pack(np.zeros((4, 64), np.int8), 2).nbytes == 4 * 64 // 4
    cap = g["capacity"]
    for bits, gb in cap["bits_to_gb"].items():
        assert abs(cap["n_params"] * int(bits) / 8 / 1e9 - gb) < 1e-9


# ---------------------------------------------------------------- products

@pytest.mark.parametrize("seed", range(5))
def test_int_dot_bruteforce_4x4(seed):
    g = np.random.default_rng(seed)
    w = g.integers(-127, 128, size=(4, 4)).astype(np.int8)
    x = g.integers(-127, 128, size=4).astype(np.int8)
    want = [sum(int(w[i, j]) * int(x[j]) for j in range(4)) for i in range(4)]
    assert oracle.int_dot_bruteforce(w, x).tolist() == want
    assert oracle.int_dot_exact(w, x).tolist() == want
    xm = g.integers(-127, 128, size=(3, 4)).astype(np.int8)
    gm = oracle.int_gemm_exact(xm, w)
    assert gm.tolist() == [[sum(int(xm[a, j]) * int(w[b, j]) for j in range(4)) for b in range(4)] for a in range(3)]


def test_int_dot_extremes_exact():
    k = 11008
    w = np.full((2, k), -127, np.int8)
    w[1] = 127
    x = np.full(k, -127, np.int8)
    assert oracle.int_dot_exact(w, x).tolist() == [k * 127 * 127, -k * 127 * 127]
    with pytest.raises(OverflowError):
        _check_exact(2 ** 40, 128, 128)


def test_unit_scale_reduces_to_integer_matmul():
    # integer-valued W and x whose largest magnitude is 127: s = 1, the codes
    # are the values themselves and the quantized GEMV is the textbook product
    g = np.random.default_rng(7)
    w = g.integers(-127, 128, size=(6, 32)).astype(np.float32)
    w[:, 0] = 127
    x = g.integers(-127, 128, size=32).astype(np.float32)
    x[3] = -127
    wq, s_w = oracle.quantize_absmax(w, per_row=True)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    assert np.all(s_w == 1) and s_x[0] == 1
    acc = oracle.int_dot_exact(wq, xq)
    assert np.array_equal(acc, (w.astype(np.int64) @ x.astype(np.int64)))
    assert np.array_equal(oracle.y_w8a8(acc, s_w, s_x), acc.astype(np.float64))


def test_float_references_against_fractions():
    g = np.random.default_rng(11)
    w = (g.standard_normal((4, 4)) * 0.02).astype(np.float32)
    x = g.standard_normal(4).astype(np.float32)
    wq, s_w = oracle.quantize_absmax(w, per_row=True)
    xq, s_x = oracle.quantize_absmax(x, per_row=False)
    acc = oracle.int_dot_exact(wq, xq)
    y = oracle.y_w8a8(acc, s_w, s_x)
    for i in range(4):
        ex = sum(Fraction(int(wq[i, j])) / Fraction(float(s_w[i])) * Fraction(int(xq[j])) / Fraction(float(s_x[0]))
                 for j in range(4))
        assert abs(Fraction(float(y[i])) - ex) <= abs(ex) * Fraction(1, 10 ** 14)
    xb = synth.to_bf16_bits(x)
    y16 = oracle.y_w8a16(wq, s_w, xb)
    xf = oracle.bf16_bits_to_f32(xb)
    for i in range(4):
        ex = sum(Fraction(int(wq[i, j])) / Fraction(float(s_w[i])) * Fraction(float(xf[j])) for j in range(4))
        assert abs(Fraction(float(y16[i])) - ex) <= abs(ex) * Fraction(1, 10 ** 14)


def test_neuron_example_dense_reference():
    ex = _golden("small_examples.json")["neuron"]
    w = np.array([ex["W"]], np.float64)
    # relative_method_error's dense product W x: a quantized output equal to
    # the dense one has zero error; the printed z values pin the product
    for xs, z in ((ex["x"], ex["z"]), (ex["x_prime"], ex["z_prime"])):
        x = np.array(xs, np.float64)
        y = np.array([z - ex["b"]])
        assert oracle.relative_method_error(y, w, x) < 1e-12


def test_sign_residual_and_ternary_outputs():
    g = np.random.default_rng(5)
    sign = np.where(g.random((3, 8)) < 0.5, -1, 1).astype(np.int8)
    rq = g.integers(-127, 128, size=(3, 8)).astype(np.int8)
    alpha = np.array([0.5, 0.25, 2.0], np.float32)
    s_r = np.array([2.0, 4.0, 0.5], np.float32)
    xb = synth.to_bf16_bits(g.standard_normal(8).astype(np.float32))
    xf = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    y = oracle.y_sign_residual(sign, alpha, rq, s_r, xb)
    for i in range(3):
        ex = sum(Fraction(float(alpha[i])) * int(sign[i, j]) * Fraction(float(xf[j])) +
                 Fraction(int(rq[i, j])) / Fraction(float(s_r[i])) * Fraction(float(xf[j])) for j in range(8))
        assert abs(Fraction(float(y[i])) - ex) <= abs(ex) * Fraction(1, 10 ** 14)
    acc = np.array([10, -3, 0], np.int64)
    yt = oracle.y_ternary(acc, np.float32(0.5), np.array([4.0], np.float32))
    assert yt.tolist() == [1.25, -0.375, 0.0]


def test_prefill_reference_linearity():
    wl = synth.prefill_outlier(m=16, k=256, n=32, n_out=4, seed=5)
    w, xb, idx = wl.tensors["w"], wl.tensors["x_bf16"], wl.tensors["idx"]
    xq, s_x, xo = oracle.outlier_split_quantize(xb, idx)
    wq, s_w = oracle.quantize_absmax(w, per_row=True)
    wo = oracle.gather_outlier_weights(w, idx)
    acc = oracle.int_gemm_exact(xq, wq)
    y = oracle.y_prefill(acc, s_x, s_w, xo, wo)
    y_int = oracle.y_prefill(acc, s_x, s_w, xo[:, :0], wo[:, :0])
    y_out = oracle.y_prefill(np.zeros_like(acc), s_x, s_w, xo, wo)
    assert np.allclose(y, y_int + y_out, rtol=1e-14, atol=1e-14)
    # the outlier path alone is the bf16 product over the gathered channels
    assert np.allclose(y_out, oracle.bf16_bits_to_f32(xo).astype(np.float64) @
                       oracle.bf16_bits_to_f32(wo).astype(np.float64).T, rtol=1e-14)
    # outlier columns of Xq are zero, so the int8 part ignores those channels
    acc2 = oracle.int_gemm_exact(xq[:, np.setdiff1d(np.arange(256), idx)],
                                 wq[:, np.setdiff1d(np.arange(256), idx)])
    assert np.array_equal(acc, acc2)
    # the split recovers the unquantized product far better than plain per-token int8
    x = oracle.bf16_bits_to_f32(xb).astype(np.float64)
    y_full = x @ w.astype(np.float64).T
    xq_plain, s_plain = oracle.quantize_absmax(oracle.bf16_bits_to_f32(xb), per_row=True)
    y_plain = oracle.int_gemm_exact(xq_plain, wq) / (s_plain[:, None].astype(np.float64) * s_w[None, :])
    e_split = np.linalg.norm(y - y_full) / np.linalg.norm(y_full)
    e_plain = np.linalg.norm(y_plain - y_full) / np.linalg.norm(y_full)
    assert e_split < e_plain / 3


def test_normwise_error():
    assert oracle.normwise_error([1.0, 2.0], [1.0, 2.0]) == 0.0
    assert abs(oracle.normwise_error([1.0, 2.1], [1.0, 2.0]) - 0.05) < 1e-12


def test_batched_weight_only_reference():
    """The M-token product: each token row is the batch-1 product (itself
    pinned above against exact rationals), the layout is [M][N], an exact
    rational check on a tiny case, and linearity across the batch."""
    g = synth.rng(41)
    n, k, m = 5, 24, 3
    w = synth.gaussian(g, (n, k), 0.02)
    wq, s_w = oracle.quantize_absmax(w, per_row=True)
    xb = synth.to_bf16_bits(synth.gaussian(g, (m, k), 1.0))
    y = oracle.y_w8a16_batch(wq, s_w, xb)
    assert y.shape == (m, n)
    for t in range(m):
        assert np.array_equal(y[t], oracle.y_w8a16(wq, s_w, xb[t]))
    xf = synth.bf16_bits_to_f32(xb)
    for t in range(m):
        for r in range(n):
            exact = sum(Fraction(int(wq[r, c])) * Fraction(float(xf[t, c])) for c in range(k)) / Fraction(float(s_w[r]))
            assert abs(y[t, r] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))
    # reversing the batch reverses the rows of y
    assert np.array_equal(oracle.y_w8a16_batch(wq, s_w, xb[::-1]), y[::-1])
