"""CPU oracle for FP8-KV paged decode attention.

TEST INFRASTRUCTURE ONLY.  This package is the plain, slow, obviously-correct
reference that the HIP path is checked against.  Only ``tests/``,
``__graft_entry__.smoke()`` and the ``cpu_baseline`` leg of ``bench.py`` may
import it.  The product path (``decode_attention_fp8_kv_amd``) never imports,
links or calls anything here, and this package never imports the product
path: the two share no code.

Sources.  The method is described by four web pages that retell one
Cloudflare engineering post; they are cited by title and section:

* [P1] "Cloudflare tối ưu hóa Kimi và GLM trên Workers AI: Kỹ thuật nén trọng
  số và quản lý bộ nhớ đệm" (aihot.vn), section "Lượng tử hóa KV cache" and
  its throughput table.
* [P2] "ترفندهای کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU"
  (news.ditty.ir), the paragraphs on the first (KV quantization) and third
  (shared-cache protection) techniques.
* [P3] "更小、更快、更安全：大规模运行Kimi和GLM" (bittide.aicompass.dev),
  section "量化 KV 缓存".
* [P4] "Tối ưu hóa mô hình AI quy mô lớn: Cách Cloudflare vận hành Kimi và
  GLM hiệu quả" (nghungs.com), section "Bảo vệ tính toàn vẹn của KV Cache".

The pages name the cache format (FP8 e4m3 instead of BF16) but do not define
its bits; the bit-level definition is the public OCP "8-bit Floating Point
Specification (OFP8)", E4M3 encoding, cited as [OFP8].

Modules:
* ``oracle.e4m3``       -- e4m3 decode/encode and the two-rounding quantizer.
* ``oracle.paged_attn`` -- append scatter, tag/abort rule, fp64 attention.
* ``oracle.page_pool``  -- generation-tagged page allocator (alloc/free) and
  the tag-checked append.
* ``oracle.scale``      -- per-tensor amax and scale for the prefill hand-off.
* ``oracle.int4_gemv``  -- INT4 weight-only decode GEMV (group-128 scales).

Parity pins for every function live in ``tests/test_oracle_*.py``; no
function here is "parity unpinned".
"""

from . import e4m3, int4_gemv, page_pool, paged_attn, scale  # noqa: F401
