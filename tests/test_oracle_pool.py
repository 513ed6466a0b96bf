"""Pins for oracle.page_pool: hand-worked allocator cases, conservation and
generation invariants over random operation sequences, and the
use-after-free scenario the tags exist to catch ([P2] third technique; [P4]
"Bảo vệ tính toàn vẹn của KV Cache")."""

import numpy as np

from oracle import page_pool as pp
from oracle import paged_attn as pa


def _pool(batch, max_pages, num_pages):
    free_pages, free_count = pp.init(num_pages)
    return dict(counts=np.zeros(batch, np.int32), table=np.full((batch, max_pages), -1, np.int32),
                expected=np.zeros((batch, max_pages), np.uint32), tags=np.zeros(num_pages, np.uint32),
                free_pages=free_pages, free_count=free_count)


def _alloc(P, n_new):
    st, P["free_count"] = pp.alloc(np.asarray(n_new, np.int32), P["counts"], P["table"], P["expected"], P["tags"],
                                   P["free_pages"], P["free_count"])
    return st


def _free(P, release):
    st, P["free_count"] = pp.free(np.asarray(release, np.uint8), P["counts"], P["table"], P["free_pages"],
                                  P["free_count"])
    return st


def test_fresh_pool_pops_in_id_order():
    P = _pool(1, 8, 8)
    assert list(_alloc(P, [5])) == [0]
    assert list(P["table"][0, :5]) == [0, 1, 2, 3, 4]
    assert P["free_count"] == 3 and P["counts"][0] == 5
    assert list(P["tags"]) == [1, 1, 1, 1, 1, 0, 0, 0]          # handed out once: generation 1
    assert list(P["expected"][0, :5]) == [1, 1, 1, 1, 1]


def test_hand_worked_prefix_rule():
    # 8 pages; requests 2, 3, 4 -> the first two fit (5 pages), the third does not (needs 4 of 3 left).
    P = _pool(3, 6, 8)
    st = _alloc(P, [2, 3, 4])
    assert list(st) == [pp.ALLOC_OK, pp.ALLOC_OK, pp.ALLOC_NO_PAGES]
    assert list(P["table"][0, :2]) == [0, 1] and list(P["table"][1, :3]) == [2, 3, 4]
    assert P["counts"].tolist() == [2, 3, 0] and P["free_count"] == 3
    # a bad request (past max_pages) is refused and does not count against the others
    st = _alloc(P, [5, 1, 2])          # seq 0: 2 + 5 > 6 -> bad; seq 1 gets 1; seq 2 gets 2
    assert list(st) == [pp.ALLOC_BAD_REQUEST, pp.ALLOC_OK, pp.ALLOC_OK]
    assert P["table"][1, 3] == 5 and list(P["table"][2, :2]) == [6, 7] and P["free_count"] == 0
    # an earlier request that does not fit stops the later ones (prefix rule); zero-page requests are served
    P2 = _pool(3, 4, 3)
    st = _alloc(P2, [4, 1, 0])
    assert list(st) == [pp.ALLOC_NO_PAGES, pp.ALLOC_NO_PAGES, pp.ALLOC_OK]
    assert P2["free_count"] == 3 and P2["counts"].tolist() == [0, 0, 0]


def test_free_pushes_in_sequence_then_slot_order_and_lifo_reuse():
    P = _pool(3, 4, 10)
    _alloc(P, [2, 3, 1])               # seq0: 0,1  seq1: 2,3,4  seq2: 5
    _free(P, [1, 0, 1])                # push 0,1 then 5
    assert P["free_count"] == 4 + 3 and P["counts"].tolist() == [0, 3, 0]
    assert list(P["free_pages"][4:7]) == [0, 1, 5]
    _alloc(P, [0, 0, 2])               # pops the last pushed first: 5, then 1
    assert list(P["table"][2, :2]) == [5, 1]
    assert P["tags"][5] == 2 and P["tags"][1] == 2 and P["tags"][0] == 1   # second owner: generation 2


def _check_invariants(P, num_pages, owned_log):
    live = []
    for b in range(P["table"].shape[0]):
        live += list(P["table"][b, :P["counts"][b]])
    free = list(P["free_pages"][:P["free_count"]])
    assert sorted(live + free) == list(range(num_pages)), "every page is owned once or free once"
    for b in range(P["table"].shape[0]):
        for j in range(P["counts"][b]):
            p = P["table"][b, j]
            assert P["expected"][b, j] == P["tags"][p], "a live slot's recorded generation is current"
    for p in range(num_pages):
        assert P["tags"][p] == owned_log[p], "tag = number of times the page was handed out"


def test_random_operation_sequences_keep_invariants():
    rng = np.random.default_rng(5)
    for trial in range(40):
        batch, max_pages, num_pages = int(rng.integers(1, 6)), int(rng.integers(1, 9)), int(rng.integers(1, 30))
        P = _pool(batch, max_pages, num_pages)
        owned = np.zeros(num_pages, np.int64)
        for step in range(25):
            if rng.random() < 0.6:
                req = rng.integers(-1, 4, batch)
                before = P["table"].copy(); cb = P["counts"].copy()
                st = _alloc(P, req)
                for b in range(batch):
                    if st[b] == pp.ALLOC_OK:
                        for j in range(cb[b], P["counts"][b]):
                            owned[P["table"][b, j]] += 1
                    else:
                        assert P["counts"][b] == cb[b] and np.array_equal(P["table"][b], before[b])
            else:
                _free(P, rng.random(batch) < 0.5)
            _check_invariants(P, num_pages, owned)


def test_use_after_free_is_caught_by_decode_and_by_checked_append():
    # seq 0 holds pages; it is freed and its pages go to seq 1.  A reader that still uses seq 0's old
    # table row and recorded tags must abort, and an append through it must be refused.
    ps, hkv, d = 16, 1, 64
    P = _pool(2, 4, 4)
    _alloc(P, [2, 0])
    old_row = P["table"][0].copy(); old_exp = P["expected"][0].copy()
    _free(P, [1, 0])
    _alloc(P, [0, 2])                                  # seq 1 now owns seq 0's former pages
    assert set(P["table"][1, :2]) == set(old_row[:2])
    table = np.stack([old_row, P["table"][1]])
    expected = np.stack([old_exp, P["expected"][1]])
    flags = pa.abort_flags(table, np.array([20, 20]), ps, 4, P["tags"], expected)
    assert list(flags) == [pa.ABORT_TAG_MISMATCH, 0]
    kc = np.zeros((4, hkv, ps, d), np.uint8); vc = np.zeros_like(kc)
    rows = np.full((2, hkv, d), 0x3F80, np.uint16)     # bf16 1.0
    st = pp.append_checked(rows, rows, np.array([0, 1]), np.array([3, 3]), table, P["tags"], expected,
                           1.0, 1.0, kc, vc)
    assert list(st) == [pp.ROW_TAG_MISMATCH, pp.ROW_WRITTEN]
    p1 = P["table"][1, 0]
    assert np.all(kc[p1, 0, 3] == 0x38)                # 1.0 in e4m3
    assert int(np.count_nonzero(kc)) == d              # only seq 1's row was written
    # a bad destination is status 2
    st = pp.append_checked(rows[:1], rows[:1], np.array([5]), np.array([0]), table, P["tags"], expected,
                           1.0, 1.0, kc, vc)
    assert list(st) == [pp.ROW_BAD_DESTINATION]


def test_free_rules_bad_count_and_full_stack():
    P = _pool(3, 4, 6)
    _alloc(P, [2, 2, 2])                          # all 6 pages out
    P["counts"][1] = 7                            # corrupt count
    st = _free(P, [1, 1, 0])
    assert list(st) == [pp.FREE_OK, pp.FREE_BAD_COUNT, pp.FREE_OK]
    assert P["free_count"] == 2 and P["counts"].tolist() == [0, 7, 2]
    # a double free cannot overflow the stack: pretend seq 2's pages were already returned
    P["free_count"] = 5
    st = _free(P, [0, 0, 1])                      # 5 + 2 > 6 -> refused, nothing written
    assert list(st) == [0, 0, pp.FREE_STACK_FULL] and P["free_count"] == 5 and P["counts"][2] == 2


def test_corrupt_stack_entry_is_recorded_without_tag_write():
    P = _pool(1, 2, 2)
    P["free_pages"][1] = 9                         # top of the stack (next pop) holds an id outside the pool
    st = _alloc(P, [2])                           # pops 9, then page 1
    assert list(st) == [0] and list(P["table"][0]) == [9, 1]
    assert list(P["expected"][0]) == [0, 1] and list(P["tags"]) == [0, 1]
    flags = pa.abort_flags(P["table"], np.array([32]), 16, 2, P["tags"], P["expected"])
    assert list(flags) == [pa.ABORT_BAD_METADATA]


def test_tag_wraps_mod_2_32():
    P = _pool(1, 1, 1)
    P["tags"][0] = np.uint32(0xFFFFFFFF)
    _alloc(P, [1])
    assert P["tags"][0] == 0 and P["expected"][0, 0] == 0
