"""Pins of the oracle's base-3 ternary packing (five digits per byte).

Exhaustive over all 243 digit tuples: the multiply-by-3 decode returns the
digits that Python's own base-3 conversion gives, the bytes are distinct and
in range, and the rounding-up bound that makes the decode exact holds; the
vectorized packer equals the loops; byte counts are 1.6 bits per weight."""
import itertools

import numpy as np

import oracle.base3 as b3
from oracle.packing import pack as pack2


def _base3_digits(v):
    d = []
    for _ in range(5):
        v, r = divmod(v, 3)
        d.append(r)
    return d[::-1]  # leading digit first


def test_all_243_tuples_round_trip():
    seen = set()
    for digits in itertools.product((0, 1, 2), repeat=5):
        t = b3.encode_digits(digits)
        assert 0 <= t <= 255
        assert b3.decode_byte(t) == list(digits)
        v = int("".join(map(str, digits)), 3)
        assert b3.decode_byte(t) == _base3_digits(v)
        # t / 256 lies in [v / 243, v / 243 + 1/243): the decode bound
        assert 243 * t >= 256 * v and 243 * t < 256 * v + 243
        seen.add(t)
    assert len(seen) == 243
    assert b3.encode_digits((0, 0, 0, 0, 0)) == 0 and b3.encode_digits((2, 2, 2, 2, 2)) == 255


def test_vectorized_matches_loops_ragged():
    g = np.random.default_rng(31)
    for k in (5, 80, 128, 333, 1024):
        codes = g.integers(-1, 2, size=(3, k)).astype(np.int8)
        p = b3.pack_base3(codes)
        assert p.shape == (3, b3.row_bytes(k))
        assert np.array_equal(p, b3.pack_base3_loops(codes))
        assert np.array_equal(b3.unpack_base3(p, k), codes)
        assert np.array_equal(b3.unpack_base3_loops(p, k), codes)
        # padding weights are q = 0 (digit 1)
        assert np.all(b3.unpack_base3(p, b3.row_bytes(k) * 5)[:, k:] == 0)


def test_bytes_per_weight():
    assert b3.row_bytes(640) * 8 / 640 == 1.6           # k a multiple of 80: exactly 1.6 bits
    assert b3.row_bytes(4096) == 832                      # 11008 x 4096: 9,158,656 bytes
    assert 11008 * b3.row_bytes(4096) == 9158656
    assert 11008 * b3.row_bytes(4096) < pack2(np.zeros((1, 4096), np.int8), 2).size * 11008


def test_first_weight_is_leading_digit():
    # codes [1, -1, 0, 0, 0] -> digits [2, 0, 1, 1, 1] -> v = 2*81 + 0 + 9 + 3 + 1 = 175
    p = b3.pack_base3(np.array([[1, -1, 0, 0, 0]], np.int8))
    assert p.shape == (1, 16)
    assert int(p[0, 0]) == (256 * 175 + 242) // 243
