"""INT4 weight-only decode GEMV (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.

Source: [P2] "ترفندهای کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU", the
paragraph on the second technique (weight compression), and [P3]
"更小、更快、更安全：大规模运行Kimi和GLM", section "压缩模型权重": the GLM
weights are stored as 4-bit integers instead of FP8; decode is bound by the
memory bandwidth that streams the weights, so halving the weight bytes makes
decode faster, while the 4-bit values must be unpacked before they are
multiplied.  The pages fix no format.  The readings taken here (the plainest
ones that make "INT4 weights" a complete definition):

* weight-only: activations x stay BF16 [M][K], the output y is [M][N];
* each weight is a signed two's-complement 4-bit integer q in [-8, 7],
  symmetric (no zero point);
* one BF16 scale per GROUP = 128 consecutive weights along K of a row:
  w[n][k] = q[n][k] * s[n][k // 128];
* storage: row n is K/8 little-endian 32-bit words; word j holds
  k = 8j .. 8j+7, nibble i (bits 4i .. 4i+3) holds k = 8j + 2i for i < 4
  and k = 8j + 2(i-4) + 1 for i >= 4 (even k in the low half-word, odd k in
  the high half-word);
* y[m][n] = sum_k x[m][k] * w[n][k], the exact value (fp64 here; every
  product and the scale are exact in fp64 and K <= 2^16 keeps the sum's
  rounding far below any BF16 output tolerance).

These are plain numpy bit operations and one fp64 matrix product.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import bf16_bits_to_f32

GROUP = 128

# k offset (within a word's 8 weights) held by nibble i
NIBBLE_K = (0, 2, 4, 6, 1, 3, 5, 7)


def unpack(words: np.ndarray) -> np.ndarray:
    """uint32 [N][K/8] -> int8 q [N][K] (see the storage reading above)."""
    words = np.asarray(words, np.uint32)
    n, kw = words.shape
    q = np.empty((n, kw, 8), np.int8)
    for i in range(8):
        nib = ((words >> np.uint32(4 * i)) & np.uint32(0xF)).astype(np.int16)
        q[:, :, NIBBLE_K[i]] = np.where(nib >= 8, nib - 16, nib).astype(np.int8)
    return q.reshape(n, kw * 8)


def dequant(words: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """fp64 weights [N][K]: q * s[n][k // GROUP] (exact)."""
    q = unpack(words).astype(np.float64)
    s = bf16_bits_to_f32(np.asarray(scale_bits, np.uint16)).astype(np.float64)
    n, k = q.shape
    if s.shape != (n, k // GROUP):
        raise ValueError(f"scales have shape {s.shape}, expected {(n, k // GROUP)}")
    return q * np.repeat(s, GROUP, axis=1)


def gemv(x_bits: np.ndarray, words: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """y [M][N] in fp64 for BF16 activations x (given as uint16 bits [M][K])."""
    x = bf16_bits_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64)
    return x @ dequant(words, scale_bits).T


def abs_mass(x_bits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """sum_k |x[m][k]| * s[n][k // GROUP] as fp64 [M][N]: the magnitude that
    bounds a finite-precision evaluation's rounding error (|q| <= 8)."""
    x = np.abs(bf16_bits_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64))
    s = bf16_bits_to_f32(np.asarray(scale_bits, np.uint16)).astype(np.float64)
    m, k = x.shape
    xg = x.reshape(m, k // GROUP, GROUP).sum(axis=2)      # [M][K/GROUP]
    return xg @ np.abs(s).T
