"""paged_decode_attn on the GPU vs the oracle over every combination of the
choices the kernels are built or dispatched on: head_dim (64, 128), cache
dtype (FP8, BF16), GQA group at both ends of both kernel families (1 and 4:
VALU; 5 and 16: MFMA) and every supported page size (16 ... 256).  Small
ragged batches (one token, a page multiple plus a tail, one past a 64-token
tile, a longer one), a stale page in every other case; each checked like the
other parity tests: cache bytes and abort flags bit for bit, outputs within
the stated tolerance, aborted sequences' outputs untouched.
"""

import itertools

import numpy as np
import pytest

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W

from parity import compare_outputs, gpu_decode, gpu_fill, oracle_decode, oracle_fill, pool_bits, say

pytestmark = pytest.mark.gpu

GRID = list(itertools.product([64, 128], [fk.KV_FP8_E4M3, fk.KV_BF16], [1, 4, 5, 16], [16, 32, 64, 128, 256]))


@pytest.mark.parametrize("d,kv,group,ps", GRID,
                         ids=[f"d{d}-{'fp8' if kv == fk.KV_FP8_E4M3 else 'bf16'}-g{g}-ps{ps}" for d, kv, g, ps in GRID])
def test_every_built_combination(gpu_device, d, kv, group, ps):
    i = GRID.index((d, kv, group, ps))
    hkv = 2
    lengths = [1, 3 * ps + 17, 64 * 5 + 1, 900]
    mismatch = [(2, 1)] if i % 2 else []
    say(f"grid case {i}: d={d} kv={kv} group={group} ps={ps} lengths={lengths} mismatch={mismatch}")
    w = W.make_custom(lengths, hkv * group, hkv, d, ps, seed=5000 + i, mismatch=mismatch)
    kc, vc = gpu_fill(w, kv, gpu_device)
    okc, ovc = oracle_fill(w, kv)
    assert np.array_equal(pool_bits(kc), okc), "K cache bytes differ from the oracle"
    assert np.array_equal(pool_bits(vc), ovc), "V cache bytes differ from the oracle"
    out, flags, _ = gpu_decode(w, kv, kc, vc, gpu_device)
    ref, rflags = oracle_decode(w, kv, okc, ovc)
    assert np.array_equal(flags, rflags), f"abort flags {flags} != oracle {rflags}"
    assert rflags.tolist() == ([0, 0, 1, 0] if mismatch else [0, 0, 0, 0])
    assert fk.paged_decode_attn_path(hkv * group, hkv) == (1 if group >= 5 else 0)
    compare_outputs(out, ref, flags)
