"""paged_decode_attn_noalloc (the decode with the library's fixed device
scratch as its workspace, for callers that cannot allocate) against
paged_decode_attn with a workspace of its own, through the C ABI.

Two calls in a row on the same device scratch, the second with a smaller
input of another shape (so it runs over what the first left in the
scratch): each must give abort flags bit-exact and outputs bit-identical to
the workspace entry point's (the same kernels and schedule), and match the
oracle to the stated tolerance; aborted sequences' outputs stay untouched.
A size whose workspace exceeds the scratch is refused before any launch.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W

from parity import OUT_SENTINEL, compare_outputs, gpu_fill, oracle_decode, oracle_fill, say

pytestmark = pytest.mark.gpu

FP8, BF16 = fk.KV_FP8_E4M3, fk.KV_BF16


def _call(w, kv, kc, vc, dev, noalloc, exp=None):
    exp = w.expected_tags if exp is None else exp
    out = torch.full(tuple(w.q.shape), 0, dtype=torch.int16, device=dev)
    out.fill_(OUT_SENTINEL)
    out = out.view(torch.bfloat16)
    flags = torch.full((w.batch,), 0xEE, dtype=torch.uint8, device=dev)
    args = (w.q.to(dev).contiguous(), kc, vc, torch.from_numpy(w.page_table).to(dev),
            torch.from_numpy(w.seq_lens.astype(np.int32)).to(dev), out, flags)
    kw = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale,
              page_tags=torch.from_numpy(w.page_tags.view(np.int32)).to(dev),
              expected_tags=torch.from_numpy(np.ascontiguousarray(exp).view(np.int32)).to(dev),
              softmax_scale=w.softmax_scale)
    if noalloc:
        fk.paged_decode_attn_noalloc(*args, **kw)
    else:
        ws = fk.alloc_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.max_pages,
                                device=dev)
        ws.fill_(0xA5)
        fk.paged_decode_attn(*args, ws, **kw)
    torch.cuda.synchronize(dev)
    return W.bits_u16(out), flags.cpu().numpy()


def test_noalloc_matches_the_workspace_entry_point(gpu_device):
    dev = gpu_device
    cases = [
        # larger input first: 6 sequences at the main shape, long ones split over many waves, one stale page
        (W.make_custom([9000, 4097, 700, 64, 20000, 1], 64, 8, 128, 64, seed=41, mismatch=[(3, 0)]), FP8),
        # then a smaller input of another shape (group 4, head_dim 64, 16-token pages, VALU family, BF16)
        (W.make_custom([300, 45], 8, 2, 64, 16, seed=42, mismatch=[]), BF16),
    ]
    for i, (w, kv) in enumerate(cases):
        say(f"noalloc call {i}: B={w.batch} hq={w.num_q_heads} hkv={w.num_kv_heads} d={w.head_dim} kv={kv}")
        need = fk.paged_decode_attn_workspace_size(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim,
                                                   w.page_size, w.max_pages)
        assert 0 < need <= fk.NOALLOC_SCRATCH_BYTES
        kc, vc = gpu_fill(w, kv, dev)
        got, gflags = _call(w, kv, kc, vc, dev, noalloc=True)
        want, wflags = _call(w, kv, kc, vc, dev, noalloc=False)
        assert np.array_equal(gflags, wflags), f"flags {gflags.tolist()} != {wflags.tolist()}"
        assert np.array_equal(got, want), "no-allocation outputs differ from the workspace entry point's"
        okc, ovc = oracle_fill(w, kv)
        ref, rflags = oracle_decode(w, kv, okc, ovc, tags_on=True)
        assert np.array_equal(gflags, rflags)
        compare_outputs(got, ref, gflags)
    assert cases[0][0].batch > cases[1][0].batch


def test_noalloc_refuses_sizes_beyond_its_scratch(gpu_device):
    dev = gpu_device
    w = W.make_custom([500, 70], 64, 8, 128, 64, seed=43, mismatch=[])
    kc, vc = gpu_fill(w, FP8, dev)
    out = torch.empty(tuple(w.q.shape), dtype=torch.bfloat16, device=dev)
    flags = torch.empty((w.batch,), dtype=torch.uint8, device=dev)
    with pytest.raises(fk.Fp8KvError) as e:   # 65535 workgroups: far more partial slots than 32 MiB
        fk.paged_decode_attn_noalloc(w.q.to(dev), kc, vc, torch.from_numpy(w.page_table).to(dev),
                                     torch.from_numpy(w.seq_lens.astype(np.int32)).to(dev), out, flags,
                                     k_scale=w.k_scale, v_scale=w.v_scale, num_blocks=65535)
    assert e.value.status == fk.ERR_SCRATCH
