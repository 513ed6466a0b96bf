"""The decode step (kv_quant_append + paged_decode_attn, or the one
paged_decode_step call) captured in a HIP graph and replayed: the library
allocates nothing, never synchronizes and issues no memset, so the calls can
be captured as they are.  Each replay
runs after eager work (new query values, output buffers refilled) and must
give bit for bit what the same calls give eagerly; the first replay is also
checked against the oracle."""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W

from parity import OUT_SENTINEL, compare_outputs, gpu_fill, oracle_decode, oracle_fill, say

pytestmark = pytest.mark.gpu

FP8 = fk.KV_FP8_E4M3


# a batch whose split segments are merged one wave per query head, and one
# long sequence whose segments spread over many waves (four per query head)
@pytest.mark.parametrize("lengths", [[3000, 700, 65, 4097, 1], [8192]], ids=["batch5", "one_long"])
@pytest.mark.parametrize("api", ["two_calls", "step_tags_on", "step_tags_off"])
def test_step_replays_in_a_hip_graph(gpu_device, lengths, api):
    dev = gpu_device
    w = W.make_custom(lengths, 64, 8, 128, 64, seed=len(lengths) + 7, mismatch=[])
    kc, vc = gpu_fill(w, FP8, dev)
    # the step's append: every sequence's last cached row once more (the same bytes)
    last = (w.ctx_pos.cpu() == torch.from_numpy(w.seq_lens.astype(np.int32))[w.ctx_seq.cpu().long()] - 1)
    idx = torch.nonzero(last).flatten()
    nk, nv = w.ctx_k.cpu()[idx].to(dev).contiguous(), w.ctx_v.cpu()[idx].to(dev).contiguous()
    ns, npos = w.ctx_seq.cpu()[idx].to(dev), w.ctx_pos.cpu()[idx].to(dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    sl = torch.from_numpy(w.seq_lens.astype(np.int32)).to(dev)
    tags = torch.from_numpy(w.page_tags.view(np.int32)).to(dev)
    exp = torch.from_numpy(np.ascontiguousarray(w.expected_tags).view(np.int32)).to(dev)
    q = w.q.to(dev).contiguous()
    ws = fk.alloc_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            w.page_table.shape[1], device=dev)
    out = torch.empty(tuple(q.shape), dtype=torch.bfloat16, device=dev)
    flags = torch.empty((w.batch,), dtype=torch.uint8, device=dev)
    out_e, flags_e = torch.empty_like(out), torch.empty_like(flags)

    tags_on = api != "step_tags_off"

    def step(o, f):
        if api == "two_calls":
            fk.kv_quant_append(nk, nv, ns, npos, pt, w.k_scale, w.v_scale, kc, vc, FP8)
            fk.paged_decode_attn(q, kc, vc, pt, sl, o, f, ws, kv_dtype=FP8, k_scale=w.k_scale, v_scale=w.v_scale,
                                 page_tags=tags, expected_tags=exp, softmax_scale=w.softmax_scale)
        else:
            fk.paged_decode_step(nk, nv, ns, npos, q, kc, vc, pt, sl, o, f, ws, kv_dtype=FP8, k_scale=w.k_scale,
                                 v_scale=w.v_scale, page_tags=tags if tags_on else None,
                                 expected_tags=exp if tags_on else None, softmax_scale=w.softmax_scale)

    side = torch.cuda.Stream(dev)
    side.wait_stream(torch.cuda.current_stream(dev))
    with torch.cuda.stream(side):
        for _ in range(2):
            step(out, flags)
    torch.cuda.current_stream(dev).wait_stream(side)
    torch.cuda.synchronize(dev)
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        step(out, flags)
    torch.cuda.synchronize(dev)

    gen = torch.Generator().manual_seed(99)
    for r in range(3):
        say(f"graph replay {r} lengths={lengths} api={api}")
        if r > 0:  # new queries: the graph reads the live buffer
            q.copy_(torch.randn(tuple(q.shape), generator=gen).to(torch.bfloat16).to(dev))
        out.view(torch.int16).fill_(OUT_SENTINEL)
        flags.fill_(0xEE)
        graph.replay()
        torch.cuda.synchronize(dev)
        step(out_e, flags_e)
        torch.cuda.synchronize(dev)
        assert torch.equal(flags, flags_e)
        assert torch.equal(out.view(torch.int16), out_e.view(torch.int16)), f"replay {r} differs from eager"
        if r == 0:
            okc, ovc = oracle_fill(w, FP8)
            ref, rflags = oracle_decode(w, FP8, okc, ovc, tags_on=tags_on)
            got_flags = flags.cpu().numpy()
            assert np.array_equal(got_flags, rflags)
            compare_outputs(W.bits_u16(out), ref, got_flags)
