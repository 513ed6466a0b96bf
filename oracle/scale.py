"""Per-tensor scale for the prefill -> decode hand-off (TEST INFRASTRUCTURE ONLY).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.

Source: [P1] "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI", section
"Lượng tử hóa KV cache", and [P3] "更小、更快、更安全：大规模运行Kimi和GLM",
section "量化 KV 缓存": prefill keeps its K/V in BF16 and decode reads an FP8
cache, so a prefill's K/V are converted once when they are handed to the
decode pool.  The pages fix neither the scale rule nor its granularity; the
reading taken here (one fp32 scale per tensor, as for the cache itself) is
the plainest one that maps the largest magnitude onto the largest e4m3
value:

    amax  = max |x| over the finite elements of the tensor (0 if none)
    scale = fp32(amax) / fp32(448)   (IEEE fp32 division), or 1.0 if amax = 0

NaNs are ignored, and so are infinities (they saturate to +-448 when
quantized with any finite scale).
"""

from __future__ import annotations

import numpy as np

from .e4m3 import bf16_bits_to_f32

E4M3_MAX = 448.0


def absmax(bits: np.ndarray) -> np.float32:
    """max |x| over the finite elements of a BF16 tensor given as uint16 bits."""
    x = bf16_bits_to_f32(np.asarray(bits, np.uint16).ravel())
    x = x[np.isfinite(x)]
    return np.float32(np.abs(x).max()) if x.size else np.float32(0.0)


def scale_from_amax(amax) -> np.float32:
    a = np.float32(amax)
    if not (a > 0):
        return np.float32(1.0)
    return np.float32(a / np.float32(E4M3_MAX))
