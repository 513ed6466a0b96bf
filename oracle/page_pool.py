"""Generation-tagged page pool: the write side of the tag check (TEST INFRASTRUCTURE ONLY).

Oracle for the page allocator that keeps the tags the decode path checks.
Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this module.

Source: [P2] "ترفندهای کلادفلر برای جا دادن مدل‌های غول‌پیکر تو GPU", third
technique, and [P4] "Tối ưu hóa mô hình AI quy mô lớn", section "Bảo vệ tính
toàn vẹn của KV Cache": every cache page carries a generation tag that
changes whenever the page is handed to a new owner, and readers compare it
with the generation they recorded before using the page.  The pages fix no
allocator; the readings taken here (plainest ones consistent with that):

* The free pages form a stack of page ids.  A fresh pool holds every page,
  arranged so that successive pops return 0, 1, 2, ...
* ``alloc``: sequence b asks for n_new[b] more pages.  A request is valid if
  n_new[b] >= 0, 0 <= page_counts[b] and page_counts[b] + n_new[b] <=
  max_pages (else status 2, nothing changes for b).  Valid requests are
  served in order of b while the running total of valid requests fits in
  the free stack: request b is served iff (sum of the valid requests before
  b) + n_new[b] <= free_count at the call (else status 1).  So the served
  requests with pages are a prefix of the valid ones; a request that does
  not fit also stops every later one, except that a request for zero pages
  is always served.
* A served request pops its pages in order; each popped page's tag is
  incremented (mod 2^32) -- the page changes owner, so its generation
  changes -- and the new tag is recorded as the sequence's expected tag for
  that slot.
* A popped id outside [0, num_pages) (a corrupt stack) is recorded as is,
  with expected tag 0 and no tag change; the decode's page check then
  flags it.
* ``free``: every sequence with release[b] != 0 pushes its pages back, in
  order of b then slot, and holds 0 pages afterwards (status 0).  A count
  outside [0, max_pages] is status 2 (nothing happens).  Like alloc, the
  pushes are a prefix: sequence b is pushed iff free_count + (pages of the
  valid released sequences before b) + its count <= num_pages (else status
  1), so a double free can never overflow the stack.  Tags do not change on
  free (they change when the page is handed out again); the freed
  sequence's table row is left as it was, so a reader that still uses it
  fails the tag check once the page has a new owner.
* ``append_checked``: kv_quant_append that writes a row only if its page's
  current tag equals the tag its sequence recorded for that slot
  (row status 0 written, 1 tag mismatch, 2 invalid destination).

Every function works in place on numpy arrays and loops in plain Python --
the obvious sequential definition.
"""

from __future__ import annotations

import numpy as np

from . import paged_attn as pa

ALLOC_OK = 0
ALLOC_NO_PAGES = 1
ALLOC_BAD_REQUEST = 2

FREE_OK = 0
FREE_STACK_FULL = 1
FREE_BAD_COUNT = 2

ROW_WRITTEN = 0
ROW_TAG_MISMATCH = 1
ROW_BAD_DESTINATION = 2


def init(num_pages: int):
    """A fresh pool: (free_pages [num_pages] int32, free_count)."""
    free_pages = np.arange(num_pages - 1, -1, -1, dtype=np.int32)  # top of the stack = last entry = page 0
    return free_pages, num_pages


def alloc(n_new, page_counts, page_table, expected_tags, page_tags, free_pages, free_count):
    """Serve page requests in order (see module docstring).  Updates the
    arrays in place; returns (status uint8 [batch], new free_count)."""
    batch, max_pages = page_table.shape
    free_count = min(max(int(free_count), 0), len(free_pages))  # a count outside the stack is clamped
    status = np.zeros(batch, np.uint8)
    valid = []
    for b in range(batch):
        r, c = int(n_new[b]), int(page_counts[b])
        if r < 0 or c < 0 or c + r > max_pages:
            status[b] = ALLOC_BAD_REQUEST
        else:
            valid.append(b)
    before = 0
    served = []
    for b in valid:
        r = int(n_new[b])
        if r == 0 or before + r <= free_count:
            served.append((b, before))
        else:
            status[b] = ALLOC_NO_PAGES
        before += r
    taken = 0
    for b, start in served:
        r, c = int(n_new[b]), int(page_counts[b])
        for k in range(r):
            p = int(free_pages[free_count - 1 - (start + k)])
            page_table[b, c + k] = p
            if 0 <= p < len(page_tags):
                page_tags[p] = np.uint32((int(page_tags[p]) + 1) & 0xFFFFFFFF)
                expected_tags[b, c + k] = page_tags[p]
            else:
                expected_tags[b, c + k] = 0
        page_counts[b] = c + r
        taken += r
    return status, free_count - taken


def free(release, page_counts, page_table, free_pages, free_count):
    """Return the pages of every released sequence (see module docstring).
    Updates the arrays in place; returns (status uint8 [batch], new free_count)."""
    batch, max_pages = page_table.shape
    num_pages = len(free_pages)
    free_count = min(max(int(free_count), 0), num_pages)  # a count outside the stack is clamped
    status = np.zeros(batch, np.uint8)
    before = 0
    pushed = []
    for b in range(batch):
        if not release[b]:
            continue
        c = int(page_counts[b])
        if c < 0 or c > max_pages:
            status[b] = FREE_BAD_COUNT
            continue
        if free_count + before + c <= num_pages:
            pushed.append((b, before))
        else:
            status[b] = FREE_STACK_FULL
        before += c
    top = free_count
    for b, start in pushed:
        c = int(page_counts[b])
        for k in range(c):
            free_pages[free_count + start + k] = page_table[b, k]
        page_counts[b] = 0
        top += c
    return status, top


def append_checked(k_new, v_new, row_seq, row_pos, page_table, page_tags, expected_tags, k_scale, v_scale,
                   k_cache, v_cache, kv_dtype=pa.KV_FP8_E4M3):
    """kv_quant_append that refuses rows whose page changed owner; returns the row status [n_rows]."""
    n_rows = len(row_seq)
    batch, max_pages = page_table.shape
    num_pages = k_cache.shape[0]
    page_size = k_cache.shape[2]
    status = np.full(n_rows, ROW_BAD_DESTINATION, np.uint8)
    ok = np.zeros(n_rows, bool)
    for i in range(n_rows):
        s, pos = int(row_seq[i]), int(row_pos[i])
        if s < 0 or s >= batch or pos < 0 or pos >= max_pages * page_size:
            continue
        j = pos // page_size
        p = int(page_table[s, j])
        if p < 0 or p >= num_pages:
            continue
        if int(page_tags[p]) != int(expected_tags[s, j]):
            status[i] = ROW_TAG_MISMATCH
            continue
        status[i] = ROW_WRITTEN
        ok[i] = True
    idx = np.nonzero(ok)[0]
    if idx.size:
        pa.append(k_new[idx], v_new[idx], np.asarray(row_seq)[idx], np.asarray(row_pos)[idx], page_table,
                  k_scale, v_scale, k_cache, v_cache, kv_dtype)
    return status
