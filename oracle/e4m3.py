"""Oracle: FP8 e4m3 codec and the per-tensor-scale quantizer (CPU, numpy).

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import it.

What the pages fix: the KV cache is held as 8-bit floating point in the e4m3
layout instead of 16-bit BF16, halving its size ([P1] section "Lượng tử hóa KV
cache"; [P3] section "量化 KV 缓存"; [P2] first technique).  The pages do not
spell out the bits; they are the OCP OFP8 E4M3 encoding [OFP8]:

* 1 sign bit, 4 exponent bits (bias 7), 3 mantissa bits;
* exponent field 0 encodes subnormals  (-1)^S * (M/8) * 2^-6;
* exponent field 1..15 encodes normals (-1)^S * (1 + M/8) * 2^(E-7);
* there are no infinities; S.1111.111 (0x7F, 0xFF) is NaN, so the largest
  finite magnitude is S.1111.110 = 448.

Encoding (the quantizer's second rounding) is round-to-nearest, ties to the
even code, saturating: magnitudes above 448 (and +-inf) become +-448, as in
OFP8's saturating conversion mode.  Readings the pages leave open, listed
here and in the design notes: every NaN input encodes to 0x7F (a NaN's sign
carries no meaning, and IEEE arithmetic does not fix the sign of a NaN that
comes out of the quantizer's division); negative inputs that round to zero
keep their sign (0x80).

Quantization uses one fp32 scale per tensor (one for K, one for V):
``code = encode(fp32(x) / fp32(scale))`` -- an IEEE fp32 division (correctly
rounded), then the e4m3 rounding above.  That is two roundings; dequantized
values are ``decode(code) * scale``.
"""

from __future__ import annotations

import numpy as np

E4M3_MAX = 448.0
E4M3_MIN_NORMAL = 2.0 ** -6
E4M3_MIN_SUBNORMAL = 2.0 ** -9
NAN_CODE = 0x7F
MAX_CODE = 0x7E


def _decode_one(code: int) -> float:
    """Value of one e4m3 byte by the OFP8 E4M3 field definitions."""
    sign = -1.0 if code & 0x80 else 1.0
    exp_field = (code >> 3) & 0xF
    man_field = code & 0x7
    if exp_field == 0xF and man_field == 0x7:
        return float("nan")
    if exp_field == 0:
        return sign * (man_field / 8.0) * 2.0 ** -6
    return sign * (1.0 + man_field / 8.0) * 2.0 ** (exp_field - 7)


_LUT = np.array([_decode_one(c) for c in range(256)], dtype=np.float64)


def decode_lut() -> np.ndarray:
    """float64[256]: the value of every e4m3 code (NaN at 0x7F and 0xFF)."""
    return _LUT.copy()


def decode(codes) -> np.ndarray:
    """Exact float64 values of an array of e4m3 bytes."""
    return _LUT[np.asarray(codes, dtype=np.uint8)]


def encode(v) -> np.ndarray:
    """Round fp32 values to e4m3 codes: nearest, ties to even, saturating.

    Every step below is exact in float64 (the inputs are fp32), so the only
    rounding is the explicit round-half-to-even of the 3-bit mantissa.
    """
    v = np.asarray(v, dtype=np.float32)
    with np.errstate(invalid="ignore"):
        a = np.abs(v.astype(np.float64))
    sign = (np.signbit(v).astype(np.uint8) << 7).astype(np.uint8)
    code = np.zeros(v.shape, dtype=np.int64)

    is_nan = np.isnan(a)
    saturate = ~is_nan & (a >= E4M3_MAX)
    subnormal = ~is_nan & (a < E4M3_MIN_NORMAL)
    normal = ~is_nan & ~saturate & ~subnormal

    # Below 2^-6 the grid is the multiples of 2^-9 (codes 0..7); rounding up
    # to 8 lands exactly on code 0x08 = 2^-6, the smallest normal.
    code[subnormal] = np.rint(a[subnormal] * 512.0).astype(np.int64)

    # Normal range: a = 2^e * (1 + f/8) with f in [0, 8).
    frac, exp2 = np.frexp(a[normal])          # a = frac * 2^exp2, frac in [0.5, 1)
    e = exp2.astype(np.int64) - 1             # a = (2 frac) * 2^e, 2 frac in [1, 2)
    mant = np.rint((2.0 * frac - 1.0) * 8.0).astype(np.int64)
    carry = mant == 8                         # rounded up into the next binade
    e = e + carry
    mant = np.where(carry, 0, mant)
    code[normal] = ((e + 7) << 3) | mant

    code[saturate] = MAX_CODE
    out = np.asarray(code.astype(np.uint8) | sign, dtype=np.uint8)
    return np.where(is_nan, np.uint8(NAN_CODE), out).astype(np.uint8)


def bf16_bits_to_f32(bits) -> np.ndarray:
    """BF16 bit patterns (uint16) -> float32 values (exact: zero-extend)."""
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32)


def quantize(x_bf16_bits, scale: float) -> np.ndarray:
    """BF16 values -> e4m3 codes with one fp32 scale: encode(fp32(x) / scale).

    The scale is an fp32 value and the quotient an fp32 value: numpy's float32
    division (IEEE, correctly rounded) -- deliberately not a float64 or exact
    division -- and that fp32 quotient is what gets rounded to e4m3.
    """
    x = bf16_bits_to_f32(x_bf16_bits)
    s = np.float32(scale)
    with np.errstate(over="ignore", invalid="ignore", divide="ignore"):
        q = (x / s).astype(np.float32)
    return encode(q)


def dequantize(codes, scale: float) -> np.ndarray:
    """e4m3 codes -> float64 values times the fp32 scale (exact in float64)."""
    return decode(codes) * float(np.float32(scale))
