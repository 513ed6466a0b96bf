"""Pins for the INT4 weight-only GEMV oracle (oracle/int4_gemv.py).

Each check comes from something other than the oracle's own code: words and
values decoded by hand from the storage reading, a pure-Python second
implementation that extracts nibbles by integer division, closed forms
(one-hot activations, constant codes) and linearity in one group's scale.
"""

import numpy as np
import pytest

from oracle import int4_gemv as i4


def _bf16(vals):
    return (np.asarray(vals, np.float32).view(np.uint32) >> 16).astype(np.uint16)


def test_unpack_hand_decoded_words():
    # nibble i holds k = 2i (i < 4) or 2(i-4)+1 (i >= 4); values are two's complement
    words = np.array([[0x76543210, 0x89ABCDEF, 0x00000008, 0x80000000, 0x0000F000, 0x00070000]], np.uint32)
    q = i4.unpack(words)
    assert q.dtype == np.int8 and q.shape == (1, 48)
    assert q[0, 0:8].tolist() == [0, 4, 1, 5, 2, 6, 3, 7]
    assert q[0, 8:16].tolist() == [-1, -5, -2, -6, -3, -7, -4, -8]
    assert q[0, 16:24].tolist() == [-8, 0, 0, 0, 0, 0, 0, 0]
    assert q[0, 24:32].tolist() == [0, 0, 0, 0, 0, 0, 0, -8]        # nibble 7 -> k = 7
    assert q[0, 32:40].tolist() == [0, 0, 0, 0, 0, 0, -1, 0]        # nibble 3 -> k = 6
    assert q[0, 40:48].tolist() == [0, 7, 0, 0, 0, 0, 0, 0]         # nibble 4 -> k = 1


def _brute(x_bits, words, scale_bits):
    """Second implementation in plain Python: nibbles by integer division,
    values from the bf16 bit fields, sums in Python floats (exact enough at
    these sizes: every term is a dyadic rational with few bits)."""
    from fractions import Fraction

    def bf16(b):
        b = int(b)
        sign = -1 if b & 0x8000 else 1
        e = (b >> 7) & 0xFF
        f = b & 0x7F
        if e == 0:
            return sign * Fraction(f, 128) * Fraction(2) ** -126
        return sign * (1 + Fraction(f, 128)) * Fraction(2) ** (e - 127)

    m_, k_ = x_bits.shape
    n_ = words.shape[0]
    y = [[Fraction(0)] * n_ for _ in range(m_)]
    for n in range(n_):
        for j in range(k_ // 8):
            word = int(words[n, j])
            for i in range(8):
                nib = (word // 16 ** i) % 16
                q = nib - 16 if nib > 7 else nib
                k = 8 * j + (2 * i if i < 4 else 2 * (i - 4) + 1)
                w = q * bf16(scale_bits[n, k // 128])
                for m in range(m_):
                    y[m][n] += bf16(x_bits[m, k]) * w
    return np.array([[float(v) for v in row] for row in y])


def test_gemv_matches_pure_python_brute_force():
    rng = np.random.default_rng(5)
    m, n, k = 2, 3, 256
    x = _bf16(rng.standard_normal((m, k)))
    words = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = _bf16(rng.uniform(0.001, 0.05, size=(n, k // 128)))
    np.testing.assert_array_equal(i4.gemv(x, words, s), _brute(x, words, s))


def test_one_hot_activation_picks_one_weight():
    rng = np.random.default_rng(6)
    n, k = 5, 512
    words = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = _bf16(rng.uniform(0.5, 2.0, size=(n, k // 128)))
    sf = s.astype(np.uint32) << 16
    sv = sf.view(np.float32).astype(np.float64)
    for kk in (0, 1, 7, 8, 130, 255, 256, 511):
        x = np.zeros((1, k), np.uint16)
        x[0, kk] = 0x3F80                                       # 1.0
        y = i4.gemv(x, words, s)[0]
        j, off = divmod(kk, 8)
        i = off // 2 if off % 2 == 0 else 4 + off // 2          # nibble that holds this k
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
    for word, q in ((0x11111111, 1), (0xFFFFFFFF, -1), (0x77777777, 7), (0x88888888, -8), (0, 0)):
        words = np.full((2, k // 8), word, np.uint32)
        y = i4.gemv(x, words, s)
        g = xf.reshape(3, 3, 128).sum(axis=2)
        np.testing.assert_allclose(y[:, 0], q * (0.25 * g[:, 0] + 2.0 * g[:, 1] + 0.125 * g[:, 2]), rtol=1e-13)
        np.testing.assert_allclose(y[:, 1], q * g.sum(axis=1), rtol=1e-13)


def test_each_group_scale_applies_to_its_own_k_range_only():
    rng = np.random.default_rng(8)
    n, k = 4, 512
    x = _bf16(rng.standard_normal((2, k)))
    words = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = _bf16(rng.uniform(0.5, 2.0, size=(n, k // 128)))
    base = i4.gemv(x, words, s)
    for g in range(k // 128):
        xg = np.zeros_like(x)
        xg[:, 128 * g:128 * (g + 1)] = x[:, 128 * g:128 * (g + 1)]
        part = i4.gemv(xg, words, s)
        s2 = s.copy()
        s2[:, g] = _bf16((s[:, g].astype(np.uint32) << 16).view(np.float32) * 2)   # exact doubling
        np.testing.assert_allclose(i4.gemv(x, words, s2) - base, part, rtol=1e-12, atol=1e-12)
        # x that lives in group g does not see the other groups' scales
        s3 = s.copy()
        s3[:, [h for h in range(k // 128) if h != g]] = 0
        np.testing.assert_array_equal(i4.gemv(xg, words, s3), part)


def test_abs_mass_bounds_the_output():
    rng = np.random.default_rng(9)
    m, n, k = 3, 6, 256
    x = _bf16(rng.standard_normal((m, k)))
    words = rng.integers(0, 2 ** 32, size=(n, k // 8), dtype=np.uint64).astype(np.uint32)
    s = _bf16(rng.uniform(0.01, 0.1, size=(n, k // 128)))
    y = i4.gemv(x, words, s)
    mass = i4.abs_mass(x, s)
    assert np.all(np.abs(y) <= 8 * mass)
    # all codes -8 with non-negative x reach the bound exactly
    xp = _bf16(np.abs(rng.standard_normal((m, k))))
    yw = i4.gemv(xp, np.full((n, k // 8), 0x88888888, np.uint32), s)
    np.testing.assert_allclose(-yw, 8 * i4.abs_mass(xp, s), rtol=1e-13)


def test_scale_shape_is_checked():
    with pytest.raises(ValueError):
        i4.dequant(np.zeros((2, 32), np.uint32), np.zeros((2, 3), np.uint16))
