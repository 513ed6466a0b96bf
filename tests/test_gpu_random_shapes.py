"""paged_decode_attn on the GPU vs the oracle over a seeded random sweep of
shapes: KV heads, GQA group (both kernel families), head size, page size,
ragged lengths (including 1 token, exact page and tile multiples), tag
mismatches in random slots, both cache dtypes and several grid sizes.

The cases are drawn once from a fixed seed, so the sweep is the same on
every run; each is checked like the hand-picked shapes: cache bytes and
abort flags bit for bit, outputs within the stated tolerance, aborted
sequences' outputs untouched.
"""

import numpy as np
import pytest

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W

from parity import compare_outputs, gpu_decode, gpu_fill, oracle_decode, oracle_fill, pool_bits, say

pytestmark = pytest.mark.gpu


def _cases(n=24, seed=20261202):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4, 8]))
        group = int(rng.choice([1, 2, 3, 4, 5, 6, 7, 8, 12, 16]))
        while hkv * group > 64:          # keep the oracle's work small
            hkv //= 2
        d = int(rng.choice([64, 128]))
        ps = int(rng.choice([16, 32, 64, 128, 256]))
        b = int(rng.integers(1, 7))
        lengths = rng.integers(1, 2500, size=b)
        # special lengths: one token, a whole number of pages, of 64-token tiles, one past a tile
        for j in range(b):
            u = rng.random()
            if u < 0.15:
                lengths[j] = 1
            elif u < 0.3:
                lengths[j] = ps * int(rng.integers(1, 12))
            elif u < 0.4:
                lengths[j] = 64 * int(rng.integers(1, 30)) + 1
        mismatch = []
        if rng.random() < 0.35:
            s = int(rng.integers(0, b))
            used = -(-int(lengths[s]) // ps)
            mismatch.append((s, int(rng.integers(0, used))))
        kv = fk.KV_FP8_E4M3 if rng.random() < 0.6 else fk.KV_BF16
        nb = int(rng.choice([0, 0, 1, 3, 17, 256]))
        out.append((i, [int(x) for x in lengths], hkv * group, hkv, d, ps, mismatch, kv, nb))
    return out


CASES = _cases()


@pytest.mark.parametrize("case", CASES, ids=[f"r{c[0]}" for c in CASES])
def test_random_shape(gpu_device, case):
    i, lengths, hq, hkv, d, ps, mismatch, kv, nb = case
    say(f"random case {i}: lengths={lengths} hq={hq} hkv={hkv} d={d} ps={ps} mismatch={mismatch} "
        f"kv={kv} blocks={nb}")
    w = W.make_custom(lengths, hq, hkv, d, ps, seed=1000 + i, mismatch=mismatch)
    kc, vc = gpu_fill(w, kv, gpu_device)
    okc, ovc = oracle_fill(w, kv)
    assert np.array_equal(pool_bits(kc), okc), "K cache bytes differ from the oracle"
    assert np.array_equal(pool_bits(vc), ovc), "V cache bytes differ from the oracle"
    out, flags, _ = gpu_decode(w, kv, kc, vc, gpu_device, num_blocks=nb)
    ref, rflags = oracle_decode(w, kv, okc, ovc)
    assert np.array_equal(flags, rflags), f"abort flags {flags} != oracle {rflags}"
    assert bool(rflags.any()) == bool(mismatch), "the injected mismatch should abort exactly its sequence"
    compare_outputs(out, ref, flags)
