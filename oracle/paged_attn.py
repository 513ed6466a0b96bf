"""Oracle: paged KV append, the page-tag/abort rule and fp64 decode attention.

TEST INFRASTRUCTURE ONLY -- see ``oracle/__init__.py`` for who may import it.

Data layout (the library's convention, restated here independently):

* K and V caches are separate pools ``[num_pages][num_kv_heads][page_size][head_dim]``
  of e4m3 bytes (uint8) or BF16 bit patterns (uint16).
* ``page_table[b][j]`` (int32) is the physical page that holds tokens
  ``j*page_size .. (j+1)*page_size - 1`` of sequence ``b``.
* ``page_tags[p]`` (uint32) is the current generation of physical page ``p``;
  ``expected_tags[b][j]`` is the generation sequence ``b`` recorded when it was
  given the page in its slot ``j``.
* BF16 tensors are carried as uint16 bit patterns; numpy has no bf16 type.

What the pages fix and what is read into them:

* The cache lives in pages of one shared physical pool that many requests
  read and write; each page carries a tag that changes whenever the page is
  reallocated; the tag is compared before the page is read, and on a mismatch
  the request is aborted instead of returning wrong data ([P2] third
  technique; [P4] section "Bảo vệ tính toàn vẹn của KV Cache").  Readings:
  the expected tag is kept per (sequence, logical page); only the pages that
  hold tokens ``< seq_len`` are checked (the partial last page included);
  an aborted sequence gets no output at all.
* Abort flags are a bitmask per sequence: bit 0 (value 1) = a tag mismatch,
  bit 1 (value 2) = invalid metadata (``seq_len`` outside
  ``[1, max_pages*page_size]`` or a page id outside ``[0, num_pages)``).  The
  metadata bit is this library's own safety addition; a tag is never compared
  for an out-of-range page id.
* The cache is e4m3 with one fp32 scale per tensor, converted as it is read
  ([P1] section "Lượng tử hóa KV cache"; [P3] section "量化 KV 缓存").  The
  BF16 mode (the pages' comparison point) stores the raw BF16 values, no scale.
* Attention is ordinary single-query softmax attention per query head;
  query head ``h`` reads KV head ``h // (num_q_heads // num_kv_heads)``
  (contiguous grouped-query groups -- a reading; the pages are silent).
  ``s_t = softmax_scale * <q, k_t>`` with ``softmax_scale`` the fp32 the
  caller passes, ``p = softmax(s)``, ``o = sum_t p_t v_t``, all in float64.
"""

from __future__ import annotations

import numpy as np

from . import e4m3

KV_FP8_E4M3 = 0
KV_BF16 = 1

ABORT_TAG_MISMATCH = 1
ABORT_BAD_METADATA = 2


def _bf16_to_f64(bits) -> np.ndarray:
    return e4m3.bf16_bits_to_f32(bits).astype(np.float64)


# --------------------------------------------------------------------------
# Append: quantize new K/V rows and scatter them into pages.
# --------------------------------------------------------------------------
def append(k_new, v_new, row_seq, row_pos, page_table, k_scale, v_scale,
           k_cache, v_cache, kv_dtype=KV_FP8_E4M3):
    """Write rows into the caches in place; returns the number of rows written.

    ``k_new``/``v_new``: uint16 BF16 bits ``[n_rows][num_kv_heads][head_dim]``.
    Row ``r`` belongs to sequence ``row_seq[r]`` at token position
    ``row_pos[r]``; it lands in page ``page_table[row_seq[r]][row_pos[r] // PS]``
    at slot ``row_pos[r] % PS``.  In FP8 mode each element becomes
    ``e4m3.quantize(x, scale)`` (K with ``k_scale``, V with ``v_scale``); in
    BF16 mode the bits are copied.  A row whose sequence index, position or
    page id is out of range is skipped (reading: the append never writes
    outside the pool).  Two rows aimed at one slot are a caller error.
    """
    k_new = np.asarray(k_new, dtype=np.uint16)
    v_new = np.asarray(v_new, dtype=np.uint16)
    row_seq = np.asarray(row_seq, dtype=np.int64)
    row_pos = np.asarray(row_pos, dtype=np.int64)
    page_table = np.asarray(page_table, dtype=np.int64)
    batch, max_pages = page_table.shape
    num_pages, _, page_size, _ = k_cache.shape

    # Which rows have a valid destination.
    ok = (row_seq >= 0) & (row_seq < batch) & (row_pos >= 0) & (row_pos < max_pages * page_size)
    page = np.full(row_seq.shape, -1, dtype=np.int64)
    page[ok] = page_table[row_seq[ok], row_pos[ok] // page_size]
    ok &= (page >= 0) & (page < num_pages)
    rows = np.nonzero(ok)[0]
    page, slot = page[rows], row_pos[rows] % page_size

    if kv_dtype == KV_FP8_E4M3:
        k_val = e4m3.quantize(k_new[rows], k_scale)
        v_val = e4m3.quantize(v_new[rows], v_scale)
    else:
        k_val, v_val = k_new[rows], v_new[rows]
    # cache[page, head, slot, :] = row[head, :] for every valid row
    k_cache[page, :, slot, :] = k_val
    v_cache[page, :, slot, :] = v_val
    return int(rows.size)


# --------------------------------------------------------------------------
# Tag check: which sequences must be aborted.
# --------------------------------------------------------------------------
def abort_flags(page_table, seq_lens, page_size, num_pages,
                page_tags=None, expected_tags=None):
    """uint8[B] abort bitmask; tags ``None`` means the check is off.

    The check is optional and off unless tags are supplied ([P2] third
    technique says it is off by default).
    """
    page_table = np.asarray(page_table, dtype=np.int64)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    batch, max_pages = page_table.shape
    tags_on = page_tags is not None
    flags = np.zeros(batch, dtype=np.uint8)
    for b in range(batch):
        length = int(seq_lens[b])
        if length < 1 or length > max_pages * page_size:
            flags[b] |= ABORT_BAD_METADATA
            continue
        n_used = -(-length // page_size)
        for j in range(n_used):
            page = int(page_table[b, j])
            if not (0 <= page < num_pages):
                flags[b] |= ABORT_BAD_METADATA
                continue
            if tags_on and int(page_tags[page]) != int(expected_tags[b, j]):
                flags[b] |= ABORT_TAG_MISMATCH
    return flags


# --------------------------------------------------------------------------
# Attention.
# --------------------------------------------------------------------------
def gather_kv(cache, page_table_row, length, kv_head, kv_dtype, scale):
    """Logical rows ``0..length-1`` of one KV head as float64 ``[length][D]``."""
    page_size = cache.shape[2]
    t = np.arange(length)
    pages = np.asarray(page_table_row, dtype=np.int64)[t // page_size]
    raw = cache[pages, kv_head, t % page_size, :]
    if kv_dtype == KV_FP8_E4M3:
        return e4m3.dequantize(raw, scale)
    return _bf16_to_f64(raw)


def attend(q, k, v, softmax_scale):
    """fp64 softmax attention of query rows ``q[G][D]`` over ``k, v [L][D]``."""
    s = float(np.float32(softmax_scale)) * (q @ k.T)          # [G][L]
    s = s - s.max(axis=1, keepdims=True)
    p = np.exp(s)
    p = p / p.sum(axis=1, keepdims=True)
    return p @ v                                               # [G][D]


def decode_attention(q, k_cache, v_cache, kv_dtype, k_scale, v_scale,
                     page_table, seq_lens, softmax_scale, flags=None,
                     batch_indices=None, q_heads=None):
    """float64 ``[B][Hq][D]`` decode-attention outputs.

    ``q``: uint16 BF16 bits ``[B][Hq][D]``.  Sequences with a nonzero abort
    flag (``flags``, default: the metadata rule with tags off) are left NaN:
    the oracle produces no output for them.  ``batch_indices`` / ``q_heads``
    restrict the work to a sample (other entries stay NaN).
    """
    q = np.asarray(q, dtype=np.uint16)
    batch, num_q_heads, head_dim = q.shape
    num_kv_heads = k_cache.shape[1]
    group = num_q_heads // num_kv_heads
    page_size, num_pages = k_cache.shape[2], k_cache.shape[0]
    if flags is None:
        flags = abort_flags(page_table, seq_lens, page_size, num_pages)
    out = np.full((batch, num_q_heads, head_dim), np.nan, dtype=np.float64)
    bs = range(batch) if batch_indices is None else batch_indices
    hs = range(num_q_heads) if q_heads is None else q_heads
    for b in bs:
        if flags[b]:
            continue
        length = int(seq_lens[b])
        for g in sorted({h // group for h in hs}):
            heads = [h for h in hs if h // group == g]
            k = gather_kv(k_cache, page_table[b], length, g, kv_dtype, k_scale)
            v = gather_kv(v_cache, page_table[b], length, g, kv_dtype, v_scale)
            out[b, heads, :] = attend(_bf16_to_f64(q[b, heads, :]), k, v,
                                      softmax_scale)
    return out
