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
* y[m][n] = sum_k x[m][k] * w[n][k], the exact value (fp64 here; every
  product and the scale are exact in fp64 and K <= 2^16 keeps the sum's
  rounding far below any BF16 output tolerance).

Two storage layouts (neither is fixed by the pages):

* rows (the common checkpoint form, input of ``pack``): codes uint32
  [N][K/8], word j of row n holds k = 8j + i in nibble i (bits 4i..4i+3);
  scales BF16 [N][K/128].
* tiles (what the GEMV reads): rows padded to Np = 16 * ceil(N/16) and cut
  into tiles of 16 rows x 128 weights.  Codes uint32 [Np/16][K/128][16][16]:
  tile t, group g, row r = n - 16t, word j holds k = 128g + 8j .. +7 with
  nibble i holding k = 128g + 8j + NIBBLE_K[i] (even k in the low half-word,
  odd k in the high one).  Scales BF16 [Np/16][K/128][16].  Padding rows
  hold code 0 and scale 0.

These are plain numpy bit operations and one fp64 matrix product.
"""

from __future__ import annotations

import numpy as np

from .e4m3 import bf16_bits_to_f32

GROUP = 128

# k offset (within a word's 8 weights) held by nibble i in the tile layout
NIBBLE_K = (0, 2, 4, 6, 1, 3, 5, 7)


def _signed(nib: np.ndarray) -> np.ndarray:
    nib = nib.astype(np.int16)
    return np.where(nib >= 8, nib - 16, nib).astype(np.int8)


def unpack_rows(words: np.ndarray) -> np.ndarray:
    """Row layout codes uint32 [N][K/8] -> int8 q [N][K]."""
    words = np.asarray(words, np.uint32)
    n, kw = words.shape
    q = np.empty((n, kw, 8), np.int8)
    for i in range(8):
        q[:, :, i] = _signed((words >> np.uint32(4 * i)) & np.uint32(0xF))
    return q.reshape(n, kw * 8)


def padded_rows(n: int) -> int:
    return -(-n // 16) * 16


def unpack_tiles(tiles: np.ndarray, n: int, k: int) -> np.ndarray:
    """Tile layout codes (any shape holding Np/16*K/128*256 words) -> int8 q [N][K]."""
    g = k // GROUP
    t = np.asarray(tiles, np.uint32).reshape(padded_rows(n) // 16, g, 16, 16)   # [tile][group][row][word]
    q = np.empty((padded_rows(n) // 16, g, 16, 16, 8), np.int8)               # [tile][group][row][word][k%8]
    for i in range(8):
        q[..., NIBBLE_K[i]] = _signed((t >> np.uint32(4 * i)) & np.uint32(0xF))
    # -> [tile][row][group][word][k%8] -> rows, k = 128 g + 8 word + k%8
    return q.transpose(0, 2, 1, 3, 4).reshape(padded_rows(n), k)[:n]


def scales_from_tiles(scale_tiles: np.ndarray, n: int, k: int) -> np.ndarray:
    """Tile layout scales -> BF16 bits [N][K/128]."""
    g = k // GROUP
    s = np.asarray(scale_tiles, np.uint16).reshape(padded_rows(n) // 16, g, 16)
    return s.transpose(0, 2, 1).reshape(padded_rows(n), g)[:n]


def pack(words: np.ndarray, scale_bits: np.ndarray):
    """Row layout (codes [N][K/8], scales [N][K/128]) -> tile layout
    (codes uint32 [Np/16][K/128][16][16], scales uint16 [Np/16][K/128][16])."""
    q = unpack_rows(words)
    n, k = q.shape
    g = k // GROUP
    npad = padded_rows(n)
    qp = np.zeros((npad, k), np.int16)
    qp[:n] = q
    nib = (qp & 0xF).astype(np.uint32).reshape(npad // 16, 16, g, 16, 8)     # [tile][row][group][word][k%8]
    out = np.zeros((npad // 16, 16, g, 16), np.uint32)
    for i in range(8):
        out |= nib[..., NIBBLE_K[i]] << np.uint32(4 * i)
    sp = np.zeros((npad, g), np.uint16)
    sp[:n] = np.asarray(scale_bits, np.uint16)
    return (out.transpose(0, 2, 1, 3).copy(), sp.reshape(npad // 16, 16, g).transpose(0, 2, 1).copy())


def _x64(x_bits):
    return bf16_bits_to_f32(np.asarray(x_bits, np.uint16)).astype(np.float64)


def gemv_rows(x_bits: np.ndarray, words: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """y [M][N] in fp64 from row-layout weights."""
    q = unpack_rows(words).astype(np.float64)
    s = bf16_bits_to_f32(np.asarray(scale_bits, np.uint16)).astype(np.float64)
    if s.shape != (q.shape[0], q.shape[1] // GROUP):
        raise ValueError(f"scales have shape {s.shape}, expected {(q.shape[0], q.shape[1] // GROUP)}")
    return _x64(x_bits) @ (q * np.repeat(s, GROUP, axis=1)).T


def gemv(x_bits: np.ndarray, tiles: np.ndarray, scale_tiles: np.ndarray, n: int) -> np.ndarray:
    """y [M][N] in fp64 from tile-layout weights (the GEMV's input format)."""
    k = np.asarray(x_bits).shape[1]
    q = unpack_tiles(tiles, n, k).astype(np.float64)
    s = bf16_bits_to_f32(scales_from_tiles(scale_tiles, n, k)).astype(np.float64)
    return _x64(x_bits) @ (q * np.repeat(s, GROUP, axis=1)).T


def abs_mass(x_bits: np.ndarray, scale_bits: np.ndarray) -> np.ndarray:
    """sum_k |x[m][k]| * |s[n][k // GROUP]| as fp64 [M][N] for row-layout
    scales [N][K/128]: the magnitude that bounds a finite-precision
    evaluation's rounding error (|q| <= 8)."""
    x = np.abs(_x64(x_bits))
    s = bf16_bits_to_f32(np.asarray(scale_bits, np.uint16)).astype(np.float64)
    m, k = x.shape
    xg = x.reshape(m, k // GROUP, GROUP).sum(axis=2)      # [M][K/GROUP]
    return xg @ np.abs(s).T
