"""Pins for the oracle's e4m3 codec (CPU only).

Each test checks the oracle against something other than itself:
* landmark values printed in the OFP8 specification (golden fixture);
* structural facts of a 4-exponent/3-mantissa binary format;
* torch's ``float8_e4m3fn`` conversion (a library routine) where it applies;
* an independent nearest-value search in exact rational arithmetic;
* pinned double-rounding examples, where one-step rounding would differ.
"""

import bisect
import math
import os
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import e4m3

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _load_landmarks():
    rows = []
    with open(os.path.join(GOLDEN, "e4m3_ofp8_landmarks.txt")) as f:
        for line in f:
            line = line.strip()
            if not line or line.startswith("#"):
                continue
            code, value = line.split()
            rows.append((int(code, 16), float(value)))
    return rows


def test_landmarks_from_ofp8_table():
    lut = e4m3.decode_lut()
    rows = _load_landmarks()
    assert len(rows) == 10
    for code, value in rows:
        got = lut[code]
        if math.isnan(value):
            assert math.isnan(got), hex(code)
        else:
            assert got == value, hex(code)
            assert math.copysign(1.0, got) == math.copysign(1.0, value), hex(code)


def test_decode_structure():
    lut = e4m3.decode_lut()
    pos = lut[:0x80]
    # exactly two NaN codes, 254 finite values
    assert np.isnan(lut).sum() == 2 and np.isnan(lut[0x7F]) and np.isnan(lut[0xFF])
    # sign bit mirrors the magnitude
    for c in range(0x7F):
        assert lut[c | 0x80] == -lut[c]
    # positive codes 0..0x7E are strictly increasing: a sign-magnitude format
    assert np.all(np.diff(pos[:0x7F]) > 0)
    # within each binade the 8 values are equally spaced by 2^(E-10) ...
    for e in range(1, 16):
        vals = pos[e * 8:(e + 1) * 8] if e < 15 else pos[e * 8:e * 8 + 7]
        steps = np.diff(vals)
        assert np.all(steps == 2.0 ** (e - 7 - 3)), e
    # ... and the subnormals continue the first normal binade's spacing 2^-9
    assert np.all(np.diff(pos[0:9]) == 2.0 ** -9)
    # binade starts are consecutive powers of two from 2^-6 to 2^8
    assert [pos[e * 8] for e in range(1, 16)] == [2.0 ** (e - 7) for e in range(1, 16)]


def test_decode_matches_torch_float8_e4m3fn():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    ref = codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()
    lut = e4m3.decode_lut()
    assert np.array_equal(np.isnan(ref), np.isnan(lut))
    fin = ~np.isnan(lut)
    assert np.array_equal(ref[fin], lut[fin])
    assert np.array_equal(np.signbit(ref[fin]), np.signbit(lut[fin]))


def test_encode_roundtrips_every_finite_code():
    lut = e4m3.decode_lut()
    codes = np.arange(256)
    fin = ~np.isnan(lut)
    got = e4m3.encode(lut[fin].astype(np.float32))
    assert np.array_equal(got, codes[fin].astype(np.uint8))


def test_encode_midpoints_go_to_even_code():
    lut = e4m3.decode_lut()
    for c in range(0x7E):                       # neighbours c, c+1 (both finite)
        mid = (lut[c] + lut[c + 1]) / 2.0       # exact in float64
        assert float(np.float32(mid)) == mid    # and representable in fp32
        even = c if c % 2 == 0 else c + 1
        assert e4m3.encode(np.float32(mid)) == even, hex(c)
        assert e4m3.encode(np.float32(-mid)) == (even | 0x80), hex(c)


def test_encode_saturates_and_handles_specials():
    big = np.array([448.0, 448.5, 460.0, 464.0, 480.0, 1e9, 3.4e38, np.inf], np.float32)
    assert np.all(e4m3.encode(big) == 0x7E)
    assert np.all(e4m3.encode(-big) == 0xFE)
    specials = np.array([0.0, -0.0, 1e-30, -1e-30, 2.0 ** -10, -(2.0 ** -10)], np.float32)
    assert list(e4m3.encode(specials)) == [0x00, 0x80, 0x00, 0x80, 0x00, 0x80]
    assert e4m3.encode(np.float32(np.nan)) == 0x7F
    assert e4m3.encode(-np.float32(np.nan)) == 0x7F


# --- an independent encoder: nearest representable value, exact arithmetic ---
# candidate values come from torch's decoder, not the oracle's
_FINITE_POS = (torch.arange(0x7F, dtype=torch.int32).to(torch.uint8)
               .view(torch.float8_e4m3fn).to(torch.float64).tolist())   # 0 .. 448 ascending


def _nearest_code_exact(x: float) -> int:
    """Nearest of the 127 non-negative finite e4m3 values, ties to the even
    code, magnitudes at/above the maximum clamp to it; sign copied."""
    neg = math.copysign(1.0, x) < 0
    a = abs(x)
    if a >= 448.0:
        code = 0x7E
    else:
        i = bisect.bisect_right(_FINITE_POS, a)       # _FINITE_POS[i-1] <= a < _FINITE_POS[i]
        lo, hi = i - 1, i
        dlo = Fraction(a) - Fraction(_FINITE_POS[lo])
        dhi = Fraction(_FINITE_POS[hi]) - Fraction(a)
        if dlo < dhi:
            code = lo
        elif dhi < dlo:
            code = hi
        else:
            code = lo if lo % 2 == 0 else hi
    return code | (0x80 if neg else 0)


def _all_bf16_as_f32():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    vals = e4m3.bf16_bits_to_f32(bits)
    return vals[~np.isnan(vals)]


@pytest.mark.parametrize("scale", [1.0, 0.0288, 3.57, 2.0 ** -3, 0.5 / 448.0])
def test_quantize_all_bf16_matches_exact_nearest(scale):
    x = _all_bf16_as_f32()
    with np.errstate(over="ignore"):
        q = (x / np.float32(scale)).astype(np.float32)
    q = q[np.isfinite(q)]
    got = e4m3.encode(q)
    ref = np.array([_nearest_code_exact(float(v)) for v in q], dtype=np.uint8)
    bad = np.nonzero(got != ref)[0]
    assert bad.size == 0, [(float(q[i]), hex(got[i]), hex(ref[i])) for i in bad[:5]]


def test_encode_matches_torch_cast_in_range():
    rng = np.random.default_rng(7)
    v = np.concatenate([
        _all_bf16_as_f32(),
        rng.standard_normal(200_000).astype(np.float32) * 50,
        rng.uniform(-448, 448, 200_000).astype(np.float32),
        (rng.standard_normal(100_000) * 2.0 ** -8).astype(np.float32),
    ])
    v = v[np.isfinite(v) & (np.abs(v) <= 448.0)]
    ref = torch.from_numpy(v).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    got = e4m3.encode(v)
    assert np.array_equal(got, ref)


def test_quantize_is_two_roundings():
    # (x, scale): the exact quotient x/scale lies just above an e4m3 midpoint,
    # but its fp32 rounding lands exactly on the midpoint, which then goes to
    # the even code -- one exact rounding would pick the odd code instead.
    cases = [(3.0, 1.9199999570846558, 0x3C, 0x3D),   # quotient -> 1.5625
             (5.0, 4.210526466369629, 0x3A, 0x39)]    # quotient -> 1.1875
    for x, scale, two_step, one_step in cases:
        bits = np.array([np.float32(x).view(np.uint32) >> 16], dtype=np.uint16)
        assert e4m3.bf16_bits_to_f32(bits)[0] == x
        assert e4m3.quantize(bits, scale)[0] == two_step
        exact = Fraction(x) / Fraction(float(np.float32(scale)))
        assert _nearest_code_exact(float(exact)) == one_step  # fp64 of exact is not a tie


def test_dequantize_is_exact_product():
    rng = np.random.default_rng(3)
    codes = rng.integers(0, 256, 10_000).astype(np.uint8)
    codes = codes[(codes & 0x7F) != 0x7F]
    scale = np.float32(0.0123)
    got = e4m3.dequantize(codes, scale)
    for c, g in zip(codes[:500], got[:500]):
        assert Fraction(g) == Fraction(e4m3._decode_one(int(c))) * Fraction(float(scale))
