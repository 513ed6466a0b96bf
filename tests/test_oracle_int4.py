"""Pins for the INT4 weight-only GEMV oracle (oracle/int4_gemv.py).

Each check comes from something other than the oracle's own code: words and
values decoded by hand from the two storage readings, a pure-Python second
implementation that locates every code by the tile index formula and
extracts nibbles by integer division, closed forms (one-hot activations,
constant codes) and linearity in one group's scale.
"""

from fractions import Fraction

import numpy as np
import pytest

from oracle import int4_gemv as i4


def _bf16(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def _rand_words(rng, shape):
    return rng.integers(0, 2 ** 32, size=shape, dtype=np.uint64).astype(np.uint32)


def test_unpack_rows_hand_decoded_words():
    # row layout: nibble i holds k = 8j + i, two's complement
    words = np.array([[0x76543210, 0x89ABCDEF, 0x00000008, 0x80000000]], np.uint32)
    q = i4.unpack_rows(words)
    assert q.dtype == np.int8 and q.shape == (1, 32)
    assert q[0, 0:8].tolist() == [0, 1, 2, 3, 4, 5, 6, 7]
    assert q[0, 8:16].tolist() == [-1, -2, -3, -4, -5, -6, -7, -8]
    assert q[0, 16:24].tolist() == [-8, 0, 0, 0, 0, 0, 0, 0]
    assert q[0, 24:32].tolist() == [0, 0, 0, 0, 0, 0, 0, -8]


def test_unpack_tiles_hand_built_buffer():
    # N = 20 rows (two tiles, the second padded), K = 256 (two groups)
    n, k = 20, 256
    tiles = np.zeros((2, 2, 16, 16), np.uint32)
    tiles[0, 0, 3, 5] = 0x76543210      # row 3, k = 40..47, nibble i -> k offset (0,2,4,6,1,3,5,7)[i]
    tiles[0, 1, 0, 0] = 0x89ABCDEF      # row 0, k = 128..135
    tiles[1, 1, 3, 15] = 0x00000008     # row 19, k = 128 + 120 = 248: nibble 0 -> k 248
    tiles[1, 0, 2, 0] = 0xF0000000      # row 18, k = 0..7: nibble 7 -> k 7
    q = i4.unpack_tiles(tiles, n, k)
    assert q.shape == (20, 256)
    assert q[3, 40:48].tolist() == [0, 4, 1, 5, 2, 6, 3, 7]
    assert q[0, 128:136].tolist() == [-1, -5, -2, -6, -3, -7, -4, -8]
    assert q[19, 248] == -8 and q[19].tolist().count(0) == 255
    assert q[18, 7] == -1 and q[18].tolist().count(0) == 255
    assert np.count_nonzero(q) == 7 + 8 + 1 + 1
    s = np.arange(2 * 2 * 16, dtype=np.uint16).reshape(2, 2, 16)
    sr = i4.scales_from_tiles(s, n, k)
    assert sr.shape == (20, 2)
    assert sr[3].tolist() == [3, 19] and sr[19].tolist() == [32 + 3, 48 + 3]


def _brute_tiles(x_bits, tiles, scale_tiles, n):
    """Second implementation in plain Python: every code located by the tile
    index formula, nibbles by integer division, exact rational arithmetic."""

    def bf16(b):
        b = int(b)
        sign = -1 if b & 0x8000 else 1
        e, f = (b >> 7) & 0xFF, b & 0x7F
        if e == 0:
            return sign * Fraction(f, 128) * Fraction(2) ** -126
        return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)

    flat_w = [int(v) for v in np.asarray(tiles).ravel()]
    flat_s = [int(v) for v in np.asarray(scale_tiles).ravel()]
    m_, k_ = x_bits.shape
    groups = k_ // 128
    nib_of_offset = {0: 0, 2: 1, 4: 2, 6: 3, 1: 4, 3: 5, 5: 6, 7: 7}
    y = [[Fraction(0)] * n for _ in range(m_)]
    for row in range(n):
        t, r = divmod(row, 16)
        for k in range(k_):
            g, j, off = k // 128, (k % 128) // 8, k % 8
            word = flat_w[((t * groups + g) * 16 + r) * 16 + j]
            nib = (word // 16 ** nib_of_offset[off]) % 16
            q = nib - 16 if nib > 7 else nib
            w = q * bf16(flat_s[(t * groups + g) * 16 + r])
            for m in range(m_):
                y[m][row] += bf16(x_bits[m, k]) * w
    return np.array([[float(v) for v in r_] for r_ in y])


def test_gemv_matches_pure_python_brute_force():
    rng = np.random.default_rng(5)
    m, n, k = 2, 19, 256
    x = _bf16(rng.standard_normal((m, k)))
    tiles = _rand_words(rng, (2, 2, 16, 16))
    st = _bf16(rng.uniform(0.001, 0.05, size=(2, 2, 16)))
    np.testing.assert_array_equal(i4.gemv(x, tiles, st, n), _brute_tiles(x, tiles, st, n))


def test_pack_preserves_every_weight_and_zero_pads():
    rng = np.random.default_rng(6)
    n, k = 37, 384
    words = _rand_words(rng, (n, k // 8))
    s = _bf16(rng.uniform(0.5, 2.0, size=(n, k // 128)))
    tiles, st = i4.pack(words, s)
    assert tiles.shape == (3, 3, 16, 16) and st.shape == (3, 3, 16)
    np.testing.assert_array_equal(i4.unpack_tiles(tiles, n, k), i4.unpack_rows(words))
    np.testing.assert_array_equal(i4.scales_from_tiles(st, n, k), s)
    assert np.all(tiles[2, :, 5:, :] == 0) and np.all(st[2, :, 5:] == 0)     # rows 37..47
    # a row-layout word of codes 0..7 lands as the interleaved word 0x75316420
    w1 = np.zeros((1, 16), np.uint32)
    w1[0, 0] = 0x76543210
    t1, _ = i4.pack(w1, np.zeros((1, 1), np.uint16))
    assert int(t1[0, 0, 0, 0]) == 0x75316420


def test_row_and_tile_gemv_agree():
    rng = np.random.default_rng(11)
    n, k = 21, 512
    x = _bf16(rng.standard_normal((4, k)))
    words = _rand_words(rng, (n, k // 8))
    s = _bf16(rng.uniform(0.01, 0.1, size=(n, k // 128)))
    tiles, st = i4.pack(words, s)
    np.testing.assert_array_equal(i4.gemv(x, tiles, st, n), i4.gemv_rows(x, words, s))


def test_one_hot_activation_picks_one_weight():
    rng = np.random.default_rng(6)
    n, k = 5, 512
    words = _rand_words(rng, (n, k // 8))
    s = _bf16(rng.uniform(0.5, 2.0, size=(n, k // 128)))
    sv = (s.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    for kk in (0, 1, 7, 8, 130, 255, 256, 511):
        x = np.zeros((1, k), np.uint16)
        x[0, kk] = 0x3F80                                       # 1.0
        y = i4.gemv_rows(x, words, s)[0]
        j, i = divmod(kk, 8)
        for row in range(n):
            nib = (int(words[row, j]) >> (4 * i)) & 0xF
            q = nib - 16 if nib >= 8 else nib
            assert y[row] == q * sv[row, kk // 128]


def test_constant_codes_give_scaled_group_sums():
    rng = np.random.default_rng(7)
    k = 384
    x = _bf16(rng.standard_normal((3, k)))
    xf = (x.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    s = _bf16([[0.25, 2.0, 0.125], [1.0, 1.0, 1.0]])
    g = xf.reshape(3, 3, 128).sum(axis=2)
    for word, q in ((0x11111111, 1), (0xFFFFFFFF, -1), (0x77777777, 7), (0x88888888, -8), (0, 0)):
        words = np.full((2, k // 8), word, np.uint32)
        for y in (i4.gemv_rows(x, words, s), i4.gemv(x, *i4.pack(words, s), 2)):
            np.testing.assert_allclose(y[:, 0], q * (0.25 * g[:, 0] + 2.0 * g[:, 1] + 0.125 * g[:, 2]),
                                       rtol=1e-13)
            np.testing.assert_allclose(y[:, 1], q * g.sum(axis=1), rtol=1e-13)


def test_each_group_scale_applies_to_its_own_k_range_only():
    rng = np.random.default_rng(8)
    n, k = 4, 512
    x = _bf16(rng.standard_normal((2, k)))
    words = _rand_words(rng, (n, k // 8))
    s = _bf16(rng.uniform(0.5, 2.0, size=(n, k // 128)))
    base = i4.gemv_rows(x, words, s)
    for g in range(k // 128):
        xg = np.zeros_like(x)
        xg[:, 128 * g:128 * (g + 1)] = x[:, 128 * g:128 * (g + 1)]
        part = i4.gemv_rows(xg, words, s)
        s2 = s.copy()
        s2[:, g] = _bf16((s[:, g].astype(np.uint32) << 16).view(np.float32) * 2)   # exact doubling
        np.testing.assert_allclose(i4.gemv_rows(x, words, s2) - base, part, rtol=1e-12, atol=1e-12)
        s3 = s.copy()
        s3[:, [h for h in range(k // 128) if h != g]] = 0
        np.testing.assert_array_equal(i4.gemv_rows(xg, words, s3), part)


def test_abs_mass_bounds_the_output():
    rng = np.random.default_rng(9)
    m, n, k = 3, 6, 256
    x = _bf16(rng.standard_normal((m, k)))
    words = _rand_words(rng, (n, k // 8))
    s = _bf16(rng.uniform(0.01, 0.1, size=(n, k // 128)))
    y = i4.gemv_rows(x, words, s)
    assert np.all(np.abs(y) <= 8 * i4.abs_mass(x, s))
    xp = _bf16(np.abs(rng.standard_normal((m, k))))
    yw = i4.gemv_rows(xp, np.full((n, k // 8), 0x88888888, np.uint32), s)
    np.testing.assert_allclose(-yw, 8 * i4.abs_mass(xp, s), rtol=1e-13)


def test_scale_shape_is_checked():
    with pytest.raises(ValueError):
        i4.gemv_rows(np.zeros((1, 256), np.uint16), np.zeros((2, 32), np.uint32), np.zeros((2, 3), np.uint16))
