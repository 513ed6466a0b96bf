"""The decode kernel's work split, restated from its rules and checked for
the invariants the kernel relies on (CPU only).

Rules (as the kernel applies them per call): each sequence with T > 0 tiles
contributes num_kv_heads segments of delta + T units -- delta = 2 start
charge when the waves average at least 16 tiles, else 0 -- laid out
sequence-major; wave w of W = min(4 * num_blocks, total units) owns units
[w*TU/W, (w+1)*TU/W); a wave's range cut at segment boundaries gives its
pieces; a piece that is a whole segment is finished in the wave, any other
piece is published in the wave's partial slot 0 (when it starts at the
wave's range start) or 1, and the wave holding a segment's first tile
describes the segment's partials as (first slot, count), the others being
slot 0 of the following waves.

Invariants: every tile of every segment lies in exactly one wave's range;
no slot receives two partials; the slots a merge reads for a segment are
exactly the slots its pieces were published in.  The GPU parity tests check
the kernel's results; this covers many more length mixes and grid sizes.
"""

import random

import numpy as np
import pytest


def _check(T_list, hkv, nb, piece_units=2, min_tiles=16):
    max_waves = 4 * nb
    TT = sum(T_list) * hkv
    n_segs = sum(1 for t in T_list if t > 0) * hkv
    delta = piece_units if TT >= min_tiles * max_waves else 0
    TU = TT + delta * n_segs
    nw = min(max_waves, TU)

    def start(w):
        return w * TU // nw

    def wave_of(x):
        return ((x + 1) * nw - 1) // TU

    covered, slots, desc, published = {}, {}, {}, {}
    for w in range(nw):
        r0, r1 = start(w), start(w + 1)
        assert r1 > r0, "every wave owns at least one unit"
        carry = 0
        for b, T in enumerate(T_list):
            U = T + delta if T > 0 else 0
            excl, carry = carry, carry + U
            if not (U > 0 and excl * hkv < r1 and (excl + U) * hkv > r0):
                continue
            seq_lo = excl * hkv
            g_first = (r0 - seq_lo) // U if r0 > seq_lo else 0
            g_last = min(hkv - 1, (r1 - 1 - seq_lo) // U)
            for g in range(g_first, g_last + 1):
                seg_lo = seq_lo + g * U + delta  # unit of the segment's first tile
                lo, hi = max(seg_lo, r0), min(seg_lo + T, r1)
                if lo >= hi:
                    continue  # only the segment's start charge
                t_lo, t_hi = lo - seg_lo, hi - seg_lo
                for t in range(t_lo, t_hi):
                    assert (b, g, t) not in covered, f"tile {(b, g, t)} in two waves"
                    covered[(b, g, t)] = w
                if t_lo == 0 and t_hi == T:
                    desc[(b, g)] = (0, 0)
                    continue
                if t_lo == 0:
                    desc[(b, g)] = (2 * w + (1 if r0 < seg_lo else 0), wave_of(seg_lo + T - 1) - w + 1)
                slot = 2 * w + (0 if seg_lo + t_lo == r0 else 1)
                assert slot not in slots, f"slot {slot} written twice"
                slots[slot] = (b, g)
                published.setdefault((b, g), []).append(slot)
    n_tiles = 0
    for b, T in enumerate(T_list):
        for g in range(hkv):
            n_tiles += T
            if T == 0:
                continue
            first_slot, n = desc[(b, g)]
            if n == 0:
                assert (b, g) not in published
                continue
            assert n >= 2
            w0 = first_slot >> 1
            merge_reads = sorted([first_slot] + [2 * (w0 + a) for a in range(1, n)])
            assert sorted(published[(b, g)]) == merge_reads, f"segment {(b, g)}"
            assert max(merge_reads) < 2 * nw
    assert len(covered) == n_tiles
    return delta, nw


def _tiles(lengths):
    return [-(-int(L) // 64) for L in lengths]


def _shaped_cases():
    rng = np.random.default_rng(5)
    yield "latency", [512], 8
    yield "long", [2048] * 8, 8
    yield "conc32-like", _tiles(rng.integers(4096, 32769, 32) + 1), 8
    lens = np.clip(np.rint(rng.lognormal(np.log(12000), 1.0, 64)), 512, 65536)
    yield "conc64-like", _tiles(lens), 8
    yield "one-token sequences", [1] * 300, 8


def _random_cases(n=60):
    rng = random.Random(1)
    for i in range(n):
        b = rng.randint(1, 40)
        T = [rng.choice([0, 1, 2, rng.randint(1, 600), rng.randint(1, 40)]) for _ in range(b)]
        if sum(T) == 0:
            T[0] = 1
        yield f"random{i}", T, rng.choice([1, 2, 4, 8])


@pytest.mark.parametrize("num_blocks", [1, 3, 17, 64, 256])
def test_schedule_covers_every_tile_once_and_merges_what_it_publishes(num_blocks):
    charged = 0
    for name, T, hkv in list(_shaped_cases()) + list(_random_cases()):
        delta, _ = _check(T, hkv, num_blocks)
        charged += delta
    if num_blocks <= 64:
        assert charged > 0, "some case exercises the start charge"
