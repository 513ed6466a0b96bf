"""paged_decode_step on the GPU over a seeded random sweep: shapes, both cache
dtypes, tags on and off, several grid sizes, and appended rows that are not
only each sequence's last token -- interior tokens, a row one past a
sequence's end (written, never attended), rows with no valid destination
(skipped) and rows of sequences that the page check aborts (still written:
the step's append is not tag-checked).

Each case withholds the chosen rows from the initial fill and hands them to
the step, then requires: cache bytes bit-exact with the oracle's fill of all
rows, abort flags bit-exact, outputs bit-identical to the two calls the step
stands for (kv_quant_append, then paged_decode_attn) and within the stated
tolerance of the oracle, aborted sequences' outputs untouched.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import paged_attn as pa

from parity import OUT_SENTINEL, _gpu_pool, _np_pool, compare_outputs, oracle_decode, pool_bits, say

pytestmark = pytest.mark.gpu


def _cases(n=16, seed=20261203):
    rng = np.random.default_rng(seed)
    out = []
    for i in range(n):
        hkv = int(rng.choice([1, 2, 4]))
        group = int(rng.choice([1, 3, 4, 5, 8, 16]))
        d = int(rng.choice([64, 128]))
        ps = int(rng.choice([16, 32, 64, 128, 256]))
        b = int(rng.integers(1, 6))
        lengths = [int(x) for x in rng.integers(2, 1500, size=b)]
        mismatch = []
        if rng.random() < 0.4:
            s = int(rng.integers(0, b))
            mismatch.append((s, int(rng.integers(0, -(-lengths[s] // ps)))))
        kv = fk.KV_FP8_E4M3 if rng.random() < 0.6 else fk.KV_BF16
        tags_on = bool(rng.random() < 0.7)
        nb = int(rng.choice([0, 0, 2, 9, 64]))
        out.append((i, lengths, hkv * group, hkv, d, ps, mismatch, kv, tags_on, nb, int(rng.integers(1 << 30))))
    return out


CASES = _cases()


def _rows(w, rng):
    """Indices of the context rows the step appends (withheld from the fill), and extra rows:
    one past a sequence's end (a real slot, never attended) and two with no valid destination."""
    seq, pos = w.ctx_seq.numpy(), w.ctx_pos.numpy()
    pick = []
    for b in range(w.batch):
        idx = np.nonzero(seq == b)[0]
        pick.append(int(idx[-1]))                                  # the last token
        if len(idx) > 2 and rng.random() < 0.5:
            pick.append(int(rng.choice(idx[:-1])))                 # an interior token
    pick = np.array(sorted(set(pick)), np.int64)
    extra_seq, extra_pos = [], []
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        if L % w.page_size:                                        # the slot after the end is in a used page
            extra_seq.append(b)
            extra_pos.append(L)
            break
    extra_seq += [-1, 0]
    extra_pos += [3, w.max_pages * w.page_size]                    # bad sequence; position past the table
    return pick, np.array(extra_seq, np.int32), np.array(extra_pos, np.int32)


@pytest.mark.parametrize("case", CASES, ids=[f"s{c[0]}" for c in CASES])
def test_random_step(gpu_device, case):
    i, lengths, hq, hkv, d, ps, mismatch, kv, tags_on, nb, rseed = case
    say(f"random step {i}: lengths={lengths} hq={hq} hkv={hkv} d={d} ps={ps} mismatch={mismatch} kv={kv} "
        f"tags_on={tags_on} blocks={nb}")
    dev = gpu_device
    w = W.make_custom(lengths, hq, hkv, d, ps, seed=3000 + i, mismatch=mismatch)
    pick, xseq, xpos = _rows(w, np.random.default_rng(rseed))
    keep = np.ones(w.ctx_k.shape[0], bool)
    keep[pick] = False
    rng = np.random.default_rng(rseed + 1)
    xk = torch.from_numpy(rng.standard_normal((len(xseq), hkv, d)).astype(np.float32)).to(torch.bfloat16)
    xv = torch.from_numpy(rng.standard_normal((len(xseq), hkv, d)).astype(np.float32)).to(torch.bfloat16)
    tp = torch.from_numpy(pick)
    nk = torch.cat([w.ctx_k[tp], xk]).contiguous()
    nv = torch.cat([w.ctx_v[tp], xv]).contiguous()
    ns = torch.cat([w.ctx_seq[tp], torch.from_numpy(xseq)])
    npos = torch.cat([w.ctx_pos[tp], torch.from_numpy(xpos)])

    pt = torch.from_numpy(w.page_table).to(dev)
    lens = torch.from_numpy(w.seq_lens).to(dev)
    q = w.q.to(dev).contiguous()
    tags = torch.from_numpy(w.page_tags.view(np.int32)).to(dev) if tags_on else None
    exp = torch.from_numpy(np.ascontiguousarray(w.expected_tags).view(np.int32)).to(dev) if tags_on else None
    common = dict(kv_dtype=kv, k_scale=w.k_scale, v_scale=w.v_scale, page_tags=tags, expected_tags=exp,
                  softmax_scale=w.softmax_scale, num_blocks=nb)

    def filled():
        kc, vc = _gpu_pool(w, kv, dev)          # the same NaN-patterned pool as the oracle's
        k = torch.from_numpy(keep)
        fk.kv_quant_append(w.ctx_k[k].to(dev).contiguous(), w.ctx_v[k].to(dev).contiguous(), w.ctx_seq[k].to(dev),
                           w.ctx_pos[k].to(dev), pt, w.k_scale, w.v_scale, kc, vc, kv)
        return kc, vc

    def outputs():
        out = torch.full(tuple(w.q.shape), 0, dtype=torch.int16, device=dev)
        out.fill_(OUT_SENTINEL)
        flags = torch.full((w.batch,), 0xEE, dtype=torch.uint8, device=dev)
        ws = fk.alloc_workspace(w.batch, hq, hkv, d, ps, w.max_pages, nb, device=dev)
        ws.fill_(0xA5)
        return out.view(torch.bfloat16), flags, ws

    kc1, vc1 = filled()
    out1, flags1, ws1 = outputs()
    fk.paged_decode_step(nk.to(dev), nv.to(dev), ns.to(dev), npos.to(dev), q, kc1, vc1, pt, lens, out1, flags1, ws1,
                         **common)
    kc2, vc2 = filled()
    out2, flags2, ws2 = outputs()
    fk.kv_quant_append(nk.to(dev), nv.to(dev), ns.to(dev), npos.to(dev), pt, w.k_scale, w.v_scale, kc2, vc2, kv)
    fk.paged_decode_attn(q, kc2, vc2, pt, lens, out2, flags2, ws2, **common)
    torch.cuda.synchronize(dev)

    okc, ovc = _np_pool(w, kv)
    pa.append(W.bits_u16(w.ctx_k), W.bits_u16(w.ctx_v), w.ctx_seq.numpy(), w.ctx_pos.numpy(), w.page_table,
              w.k_scale, w.v_scale, okc, ovc, kv)
    n = pa.append(W.bits_u16(xk), W.bits_u16(xv), xseq, xpos, w.page_table, w.k_scale, w.v_scale, okc, ovc, kv)
    assert n == len(xseq) - 2, "the extra rows: one written, two without a destination"
    for name, got, want in (("step K", kc1, okc), ("step V", vc1, ovc), ("calls K", kc2, okc), ("calls V", vc2, ovc)):
        bad = np.argwhere(pool_bits(got) != want)
        if len(bad):
            say(f"{name}: {len(bad)} elements differ; first (page, head, slot, dim): {bad[:6].tolist()}")
            p0, h0, s0, d0 = bad[0]
            say(f"  got {pool_bits(got)[p0, h0, s0, :8].tolist()} want {want[p0, h0, s0, :8].tolist()}")
    assert np.array_equal(pool_bits(kc1), okc) and np.array_equal(pool_bits(vc1), ovc), "step cache bytes"
    assert np.array_equal(pool_bits(kc2), okc) and np.array_equal(pool_bits(vc2), ovc), "two-call cache bytes"
    ref, rflags = oracle_decode(w, kv, okc, ovc, tags_on=tags_on)
    f1, f2 = flags1.cpu().numpy(), flags2.cpu().numpy()
    assert np.array_equal(f1, rflags), f"step flags {f1.tolist()} != oracle {rflags.tolist()}"
    assert np.array_equal(f2, rflags)
    assert bool(rflags.any()) == (bool(mismatch) and tags_on)
    o1, o2 = W.bits_u16(out1), W.bits_u16(out2)
    assert np.array_equal(o1, o2), "step and two-call outputs differ"
    compare_outputs(o1, ref, f1)
