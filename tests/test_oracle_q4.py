"""Pins of the group-wise 4-bit (two-level scale) oracle against what the
page fixes and against brute force ([VG] 'Why Q4_K splits weights into
blocks', 'Q4_K uses two-level blocks', figs. 43-46)."""
from fractions import Fraction

import numpy as np

import oracle.q4 as q4
import synth


def _level1_codes(w, scale, lo):
    return np.clip(np.rint((np.asarray(w, np.float32) - lo) / scale), 0, 15)


def test_page_example_blocks_beat_one_shared_scale():
    # the page's row of two differently distributed halves
    row = np.array([-0.9, -0.8, 0.1, 0.2, 4.8, 5.0, 5.1, 5.2], np.float32)
    s1, m1 = q4.group_params(row[:4])
    s2, m2 = q4.group_params(row[4:])
    assert m1 == np.float32(-0.9) and m2 == np.float32(4.8)
    err_split = []
    for blk, s, m in ((row[:4], s1, m1), (row[4:], s2, m2)):
        q = _level1_codes(blk, s, m)
        assert q[np.argmin(blk)] == 0 and q[np.argmax(blk)] == 15  # the ends map to 0 and 15
        err = np.abs(q * np.float64(s) + np.float64(m) - blk)
        assert np.all(err <= np.float64(s) / 2 * (1 + 1e-6))          # at most half a step
        err_split.append(err)
    s, m = q4.group_params(row)
    err_shared = np.abs(_level1_codes(row, s, m) * np.float64(s) + np.float64(m) - row)
    # separate blocks fit each half more closely than one scale over -0.9 .. 5.2
    assert np.max(np.concatenate(err_split)) < np.max(err_shared)


def test_storage_is_144_bytes_per_256_weights():
    w = synth.gaussian(synth.rng(7), (3, 512), 0.02)
    plane, meta = q4.pack_q4k(*q4.quantize_q4k(w))
    assert plane.shape == (3, 256) and meta.shape == (3, 2, 16)
    per_super = (plane.nbytes + meta.nbytes) / (3 * 2)
    assert per_super == 144
    assert per_super * 8 / 256 == 4.5  # bits per weight


def test_codes_are_the_nearest_grid_point():
    g = synth.rng(8)
    w = synth.gaussian(g, (6, 512), 0.02)
    w[1, 100:140] *= 30.0                     # a group with outliers
    w[2, :256] = np.abs(w[2, :256])           # all-positive super-block
    w[3, 256:] = -np.abs(w[3, 256:]) - 0.05   # all-negative super-block
    codes, sc, mm, d, dmin = q4.quantize_q4k(w)
    assert codes.max() <= 15 and sc.max() <= 63 and -31 <= mm.min() and mm.max() <= 31
    S, M = q4.reconstructed_params(sc, mm, d, dmin)
    S64 = np.repeat(S.astype(np.float64), 32, axis=1)
    M64 = np.repeat(M.astype(np.float64), 32, axis=1)
    grid = np.arange(16, dtype=np.float64)[:, None, None] * S64[None] + M64[None]     # [16][N][K]
    dist = np.abs(grid - w.astype(np.float64)[None])
    best = np.min(dist, axis=0)
    chosen = np.take_along_axis(dist, codes[None].astype(np.int64), axis=0)[0]
    assert np.all(chosen <= best + 1e-6 * S64)  # brute force over all 16 levels


def test_level2_scales_cover_the_largest_group():
    w = synth.laplace(synth.rng(9), (4, 1024), 0.02)
    codes, sc, mm, d, dmin = q4.quantize_q4k(w)
    S, M = q4.reconstructed_params(sc, mm, d, dmin)
    for r in range(4):
        for b in range(4):
            blk = w[r, 256 * b:256 * (b + 1)].reshape(8, 32)
            scales = (blk.max(1) - blk.min(1)) / 15
            j = int(np.argmax(scales))
            assert sc[r, 8 * b + j] >= 62                                   # the largest uses ~all 6 bits
            assert abs(S[r, 8 * b + j] - scales[j]) <= 0.02 * scales[j]     # fp16 d, 6-bit sc
            assert np.all(np.abs(M[r, 8 * b:8 * b + 8] - blk.min(1)) <= np.float32(dmin[r, b]) / 2 * 1.001)


def test_fields6_roundtrip_exhaustive():
    for pos in range(16):
        for v in range(64):
            vals = [0] * 16
            vals[pos] = v
            assert q4.unpack_fields6(q4.pack_fields6(vals)) == vals
    vals = list(range(63, 47, -1))
    assert q4.unpack_fields6(q4.pack_fields6(vals)) == vals


def test_pack_unpack_roundtrip_and_layout():
    w = synth.gaussian(synth.rng(10), (5, 768), 0.05)
    parts = q4.quantize_q4k(w)
    plane, meta = q4.pack_q4k(*parts)
    back = q4.unpack_q4k(plane, meta)
    for a, b in zip(parts, back):
        assert np.array_equal(np.asarray(a), np.asarray(b))
    codes = parts[0]
    assert plane[2, 7] == codes[2, 14] | (codes[2, 15] << 4)  # low nibble first
    assert int.from_bytes(meta[4, 1, 12:14].tobytes(), "little") == int(parts[3][4, 1].view(np.uint16))


def test_constant_and_zero_groups():
    w = np.zeros((2, 256), np.float32)
    w[1, :] = 0.25
    codes, sc, mm, d, dmin = q4.quantize_q4k(w)
    assert not codes.any() and not sc.any()
    what = q4.dequantize_q4k(codes, sc, mm, d, dmin)
    assert np.all(what[0] == 0)
    assert np.all(np.abs(what[1] - 0.25) <= np.float64(dmin[1, 0]) / 2)


def test_product_against_exact_rationals():
    g = synth.rng(12)
    w = synth.gaussian(g, (2, 256), 0.02)
    xb = synth.to_bf16_bits(synth.gaussian(g, (256,), 1.0))
    codes, sc, mm, d, dmin = q4.quantize_q4k(w)
    y = q4.y_q4k(codes, sc, mm, d, dmin, xb)
    S, M = q4.reconstructed_params(sc, mm, d, dmin)
    x = synth.bf16_bits_to_f32(xb)
    for r in range(2):
        exact = sum((int(codes[r, k]) * Fraction(float(S[r, k // 32])) + Fraction(float(M[r, k // 32])))
                    * Fraction(float(x[k])) for k in range(256))
        assert abs(y[r] - float(exact)) <= 1e-12 * max(1.0, abs(float(exact)))


def test_vectorized_forms_match_the_per_group_loops():
    # the quantizer against group_params plus the readings, one group at a time
    w = synth.laplace(synth.rng(13), (3, 512), 0.02)
    w[0, :32] = 0.125
    codes, sc, mm, d, dmin = q4.quantize_q4k(w)
    for r in range(3):
        for b in range(2):
            blk = w[r, 256 * b:256 * (b + 1)]
            params = [q4.group_params(blk[32 * j:32 * (j + 1)]) for j in range(8)]
            d16 = np.float16(np.float32(max(p[0] for p in params) / np.float32(63)))
            dm16 = np.float16(np.float32(max(abs(p[1]) for p in params) / np.float32(31)))
            assert d[r, b] == d16 and dmin[r, b] == dm16
            for j, (scale, lo) in enumerate(params):
                s_j = 0 if d16 == 0 else int(np.clip(np.rint(np.float32(scale / np.float32(d16))), 0, 63))
                m_j = 0 if dm16 == 0 else int(np.clip(np.rint(np.float32(lo / np.float32(dm16))), -31, 31))
                assert sc[r, 8 * b + j] == s_j and mm[r, 8 * b + j] == m_j
    # the packer against the field-by-field reference
    plane, meta = q4.pack_q4k(codes, sc, mm, d, dmin)
    for r in range(3):
        for b in range(2):
            f = [int(v) for v in sc[r, 8 * b:8 * b + 8]] + [int(v) + 32 for v in mm[r, 8 * b:8 * b + 8]]
            assert meta[r, b, :12].tobytes() == q4.pack_fields6(f)
            assert q4.unpack_fields6(meta[r, b, :12].tobytes()) == f
