"""paged_decode_step on the GPU: one call that appends the step's new rows and
decodes, with the page check (tags on) run in the append's launch.

Each case runs the same seeded inputs three ways -- the step call, the two
calls it stands for (kv_quant_append, then paged_decode_attn), and the oracle
-- and requires: cache bytes bit-exact everywhere, abort flags bit-exact with
the oracle, step outputs bit-identical to the two-call outputs (same kernels,
same schedule) and within the stated tolerance of the oracle, aborted
sequences' outputs untouched.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W

from parity import OUT_SENTINEL, compare_outputs, gpu_fill, oracle_decode, oracle_fill, pool_bits, say

pytestmark = pytest.mark.gpu

FP8, BF16 = fk.KV_FP8_E4M3, fk.KV_BF16


def _inputs(w, dev, exp=None, pt=None, lens=None):
    exp = w.expected_tags if exp is None else exp
    pt = w.page_table if pt is None else pt
    lens = w.seq_lens if lens is None else lens
    return dict(q=w.q.to(dev).contiguous(), pt=torch.from_numpy(pt).to(dev),
                lens=torch.from_numpy(np.asarray(lens, np.int32)).to(dev),
                tags=torch.from_numpy(w.page_tags.view(np.int32)).to(dev),
                exp=torch.from_numpy(np.ascontiguousarray(exp).view(np.int32)).to(dev),
                nk=w.new_k.to(dev).contiguous(), nv=w.new_v.to(dev).contiguous(), ns=w.new_seq.to(dev),
                npos=w.new_pos.to(dev))


def _out_and_flags(w, dev):
    out = torch.full(tuple(w.q.shape), 0, dtype=torch.int16, device=dev)
    out.fill_(OUT_SENTINEL)
    return out.view(torch.bfloat16), torch.full((w.batch,), 0xEE, dtype=torch.uint8, device=dev)


def _ws(w, dev, num_blocks):
    ws = fk.alloc_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size, w.max_pages,
                            num_blocks, device=dev)
    ws.fill_(0xA5)
    return ws


def _case(w, kv, dev, tags_on, num_blocks=0, exp=None, pt=None, lens=None, events=False):
    x = _inputs(w, dev, exp, pt, lens)
    tags = dict(page_tags=x["tags"] if tags_on else None, expected_tags=x["exp"] if tags_on else None)
    common = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, softmax_scale=w.softmax_scale,
                  num_blocks=num_blocks, **tags)
    # the step
    kc1, vc1 = gpu_fill(w, kv, dev, include_new=False)
    out1, flags1 = _out_and_flags(w, dev)
    evs = (torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) if events else None
    fk.paged_decode_step(x["nk"], x["nv"], x["ns"], x["npos"], x["q"], kc1, vc1, x["pt"], x["lens"], out1, flags1,
                         _ws(w, dev, num_blocks), decode_events=evs, **common)
    # the two calls
    kc2, vc2 = gpu_fill(w, kv, dev, include_new=False)
    out2, flags2 = _out_and_flags(w, dev)
    fk.kv_quant_append(x["nk"], x["nv"], x["ns"], x["npos"], x["pt"], w.k_scale, w.v_scale, kc2, vc2, kv)
    fk.paged_decode_attn(x["q"], kc2, vc2, x["pt"], x["lens"], out2, flags2, _ws(w, dev, num_blocks), **common)
    torch.cuda.synchronize(dev)
    okc, ovc = oracle_fill(w, kv, include_new=True)
    assert np.array_equal(pool_bits(kc1), okc) and np.array_equal(pool_bits(vc1), ovc), "step cache bytes"
    assert np.array_equal(pool_bits(kc2), okc) and np.array_equal(pool_bits(vc2), ovc), "two-call cache bytes"
    ref, rflags = oracle_decode(w, kv, okc, ovc, tags_on=tags_on,
                                expected_tags=exp, page_table=pt, seq_lens=lens)
    f1, f2 = flags1.cpu().numpy(), flags2.cpu().numpy()
    assert np.array_equal(f1, rflags), f"step flags {f1.tolist()} != oracle {rflags.tolist()}"
    assert np.array_equal(f2, rflags)
    o1, o2 = W.bits_u16(out1), W.bits_u16(out2)
    assert np.array_equal(o1, o2), "step and two-call outputs differ"
    compare_outputs(o1, ref, f1)
    if events:
        ms = evs[0].elapsed_time(evs[1])
        assert ms > 0.0, "the decode events were not recorded around the decode kernel"
    return rflags


@pytest.mark.parametrize("kv", [FP8, BF16], ids=["fp8", "bf16"])
@pytest.mark.parametrize("tags_on", [True, False], ids=["tags_on", "tags_off"])
@pytest.mark.parametrize("num_blocks", [0, 3])
def test_step_equals_append_then_decode(gpu_device, kv, tags_on, num_blocks):
    say(f"step vs two calls kv={kv} tags_on={tags_on} blocks={num_blocks}")
    w = W.make("conc32", batch=6, context=3000)          # one new row per sequence, appended by the step
    exp = w.expected_tags.copy()
    exp[2, 5] ^= np.uint32(1)                            # a stale page in sequence 2 (tags on: abort)
    pt = w.page_table.copy()
    pt[4, 7] = -1                                        # a bad page id in sequence 4 (abort either way)
    flags = _case(w, kv, gpu_device, tags_on, num_blocks, exp=exp, pt=pt, events=(num_blocks == 0))
    assert flags.tolist() == ([0, 0, 1, 0, 2, 0] if tags_on else [0, 0, 0, 0, 2, 0])


def test_step_without_new_rows_and_with_a_single_sequence(gpu_device):
    # n_rows = 0: the step's first launch is the page check alone; one sequence: the latency shape
    say("step, no rows")
    w = W.make_custom([1000, 70, 5], 16, 2, 128, 64, seed=3, mismatch=[(1, 0)])
    for tags_on in (True, False):
        flags = _case(w, FP8, gpu_device, tags_on)
        assert flags.tolist() == ([0, 1, 0] if tags_on else [0, 0, 0])
    say("step, one long sequence")
    w = W.make("latency", context=8192)
    assert _case(w, FP8, gpu_device, True, events=True).tolist() == [0]
