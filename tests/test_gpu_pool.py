"""Generation-tagged page pool on the GPU vs the oracle: every array bit-exact.

Random sequences of page_alloc / page_free (batches beyond one 1024-request
chunk, single requests of hundreds of pages, exhausted pools, bad requests,
double frees), the tag-checked append, and the use-after-free scenario end
to end through the decode kernel.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import page_pool as pp
from oracle import paged_attn as pa

from parity import pool_bits, say

pytestmark = pytest.mark.gpu


class Pools:
    """The same pool held on the GPU and in the oracle."""

    def __init__(self, dev, batch, max_pages, num_pages):
        self.dev = dev
        fp, fc = pp.init(num_pages)
        self.o = dict(counts=np.zeros(batch, np.int32), table=np.full((batch, max_pages), -1, np.int32),
                      expected=np.zeros((batch, max_pages), np.uint32),
                      tags=np.random.default_rng(num_pages).integers(0, 2 ** 32, num_pages).astype(np.uint32),
                      free_pages=fp, free_count=fc)
        self.g = {k: torch.from_numpy(v.view(np.int32) if v.dtype == np.uint32 else v).to(dev)
                  for k, v in self.o.items() if k != "free_count"}
        self.g["free_count"] = torch.zeros(1, dtype=torch.int32, device=dev)
        self.g["free_pages"].fill_(-7)
        fk.page_pool_init(self.g["free_pages"], self.g["free_count"])

    def alloc(self, n_new):
        st_o, self.o["free_count"] = pp.alloc(np.asarray(n_new, np.int32), self.o["counts"], self.o["table"],
                                              self.o["expected"], self.o["tags"], self.o["free_pages"],
                                              self.o["free_count"])
        st = torch.full((len(n_new),), 0xEE, dtype=torch.uint8, device=self.dev)
        g = self.g
        fk.page_alloc(torch.tensor(np.asarray(n_new, np.int32), device=self.dev), g["counts"], g["table"],
                      g["expected"], g["tags"], g["free_pages"], g["free_count"], st)
        torch.cuda.synchronize()
        assert np.array_equal(st.cpu().numpy(), st_o)
        self.compare()
        return st_o

    def free(self, release):
        st_o, self.o["free_count"] = pp.free(np.asarray(release, np.uint8), self.o["counts"], self.o["table"],
                                             self.o["free_pages"], self.o["free_count"])
        st = torch.full((len(release),), 0xEE, dtype=torch.uint8, device=self.dev)
        g = self.g
        fk.page_free(torch.tensor(np.asarray(release, np.uint8), device=self.dev), g["counts"], g["table"],
                     g["free_pages"], g["free_count"], st)
        torch.cuda.synchronize()
        assert np.array_equal(st.cpu().numpy(), st_o)
        self.compare()
        return st_o

    def compare(self):
        o, g = self.o, self.g
        fc = int(g["free_count"].item())
        assert fc == o["free_count"]
        assert np.array_equal(g["free_pages"].cpu().numpy()[:fc], o["free_pages"][:fc])
        assert np.array_equal(g["counts"].cpu().numpy(), o["counts"])
        assert np.array_equal(g["table"].cpu().numpy(), o["table"])
        assert np.array_equal(g["expected"].cpu().numpy().view(np.uint32), o["expected"])
        assert np.array_equal(g["tags"].cpu().numpy().view(np.uint32), o["tags"])


@pytest.mark.parametrize("batch,max_pages,num_pages,steps", [(3, 6, 16, 30), (40, 9, 200, 25),
                                                              (1500, 3, 3000, 12), (2, 700, 1100, 10)])
def test_alloc_free_sequences_match_oracle(gpu_device, batch, max_pages, num_pages, steps):
    say(f"page pool random ops batch={batch} max_pages={max_pages} num_pages={num_pages}")
    P = Pools(gpu_device, batch, max_pages, num_pages)
    rng = np.random.default_rng(batch * 7 + max_pages)
    for step in range(steps):
        if rng.random() < 0.6:
            req = rng.integers(-1, max(2, max_pages // 2) + 1, batch)
            if max_pages > 100 and step == 0:
                req[:] = [600, 0]                      # one request of hundreds of pages
            P.alloc(req)
        else:
            P.free(rng.random(batch) < 0.5)
    # exhaust the pool, free everything, then a double free through a stale count: sequence 0 claims
    # its former pages again -- pushed only if they fit, never past the stack
    P.alloc(np.full(batch, max_pages, np.int32))
    P.free(np.ones(batch, np.uint8))
    P.o["counts"][0] = max_pages
    P.g["counts"][0] = max_pages
    rel = np.zeros(batch, np.uint8)
    rel[0] = 1
    P.free(rel)


def test_checked_append_matches_oracle(gpu_device):
    say("checked append vs oracle")
    hkv, d, ps, batch, max_pages = 2, 64, 16, 4, 4
    P = Pools(gpu_device, batch, max_pages, 16)
    P.alloc([2, 3, 1, 0])
    P.free([0, 0, 1, 0])                               # seq 2 releases its page ...
    P.alloc([0, 0, 0, 1])                              # ... and seq 3 gets it (new generation)
    stale_row = P.o["table"].copy()
    stale_row[2, 0] = P.o["table"][3, 0]               # seq 2 still points at its former page
    stale_exp = P.o["expected"].copy()
    stale_exp[2, 0] = stale_exp[3, 0] - np.uint32(1)   # with the generation it had recorded
    rng = np.random.default_rng(2)
    n = 12
    seq = np.array([0, 0, 1, 1, 2, 3, 3, 5, -1, 0, 1, 2], np.int32)
    pos = np.array([0, 17, 5, 40, 3, 2, 9, 0, 0, 70, 47, 15], np.int32)
    k = torch.randn(n, hkv, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    v = torch.randn(n, hkv, d, generator=torch.Generator().manual_seed(4)).to(torch.bfloat16)
    shape = (16, hkv, ps, d)
    kc = torch.full(shape, 0x11, dtype=torch.uint8, device=gpu_device)
    vc = torch.full(shape, 0x22, dtype=torch.uint8, device=gpu_device)
    rs = torch.full((n,), 0xEE, dtype=torch.uint8, device=gpu_device)
    fk.kv_quant_append_checked(k.to(gpu_device), v.to(gpu_device), torch.from_numpy(seq).to(gpu_device),
                               torch.from_numpy(pos).to(gpu_device), torch.from_numpy(stale_row).to(gpu_device),
                               0.05, 0.07, kc, vc, P.g["tags"],
                               torch.from_numpy(stale_exp.view(np.int32)).to(gpu_device), rs)
    torch.cuda.synchronize()
    okc = np.full(shape, 0x11, np.uint8)
    ovc = np.full(shape, 0x22, np.uint8)
    ost = pp.append_checked(W.bits_u16(k), W.bits_u16(v), seq, pos, stale_row, P.o["tags"], stale_exp, 0.05, 0.07,
                            okc, ovc)
    assert list(rs.cpu().numpy()) == list(ost)
    assert pp.ROW_TAG_MISMATCH in ost and pp.ROW_WRITTEN in ost and pp.ROW_BAD_DESTINATION in ost
    assert np.array_equal(pool_bits(kc), okc) and np.array_equal(pool_bits(vc), ovc)


def test_use_after_free_aborts_the_stale_reader(gpu_device):
    # Sequence 0 is decoded through a table row whose pages were freed and handed to sequence 1:
    # the decode must abort it (tag mismatch) and leave its output untouched, and decode 1 normally.
    say("use-after-free end to end")
    hkv, hq, d, ps, max_pages, num_pages = 2, 8, 64, 16, 4, 8
    P = Pools(gpu_device, 2, max_pages, num_pages)
    P.alloc([3, 0])
    old_row, old_exp = P.o["table"][0].copy(), P.o["expected"][0].copy()
    P.free([1, 0])
    P.alloc([0, 3])                                    # sequence 1 now owns the same pages
    assert sorted(P.o["table"][1, :3]) == sorted(old_row[:3])
    L = 40
    table = np.stack([old_row, P.o["table"][1]]).astype(np.int32)
    expected = np.stack([old_exp, P.o["expected"][1]])
    rows_k = torch.randn(L, hkv, d, generator=torch.Generator().manual_seed(8)).to(torch.bfloat16)
    rows_v = torch.randn(L, hkv, d, generator=torch.Generator().manual_seed(9)).to(torch.bfloat16)
    shape = (num_pages, hkv, ps, d)
    kc = torch.zeros(shape, dtype=torch.uint8, device=gpu_device)
    vc = torch.zeros(shape, dtype=torch.uint8, device=gpu_device)
    seq1 = torch.ones(L, dtype=torch.int32, device=gpu_device)
    pos = torch.arange(L, dtype=torch.int32, device=gpu_device)
    tags = P.g["tags"]
    exp_t = torch.from_numpy(expected.view(np.int32)).to(gpu_device)
    rs = torch.empty(L, dtype=torch.uint8, device=gpu_device)
    fk.kv_quant_append_checked(rows_k.to(gpu_device), rows_v.to(gpu_device), seq1, pos,
                               torch.from_numpy(table).to(gpu_device), 0.02, 0.02, kc, vc, tags, exp_t, rs)
    # the stale sequence 0 may not write into its former pages
    rs0 = torch.empty(L, dtype=torch.uint8, device=gpu_device)
    fk.kv_quant_append_checked(rows_k.to(gpu_device), rows_v.to(gpu_device), torch.zeros_like(seq1), pos,
                               torch.from_numpy(table).to(gpu_device), 0.02, 0.02, kc, vc, tags, exp_t, rs0)
    q = torch.randn(2, hq, d, generator=torch.Generator().manual_seed(10)).to(torch.bfloat16).to(gpu_device)
    out = torch.full((2, hq, d), 0, dtype=torch.int16, device=gpu_device)
    out.fill_(0x7FC1)
    out = out.view(torch.bfloat16)
    flags = torch.full((2,), 0xEE, dtype=torch.uint8, device=gpu_device)
    ws = fk.alloc_workspace(2, hq, hkv, d, ps, max_pages, device=gpu_device)
    fk.paged_decode_attn(q, kc, vc, torch.from_numpy(table).to(gpu_device),
                         torch.tensor([L, L], dtype=torch.int32, device=gpu_device), out, flags, ws,
                         k_scale=0.02, v_scale=0.02, page_tags=tags, expected_tags=exp_t)
    torch.cuda.synchronize()
    assert set(rs.cpu().numpy().tolist()) == {0} and set(rs0.cpu().numpy().tolist()) == {1}
    assert list(flags.cpu().numpy()) == [pa.ABORT_TAG_MISMATCH, 0]
    assert np.all(W.bits_u16(out[0].cpu()) == 0x7FC1)
    okc = np.zeros(shape, np.uint8); ovc = np.zeros(shape, np.uint8)
    pa.append(W.bits_u16(rows_k), W.bits_u16(rows_v), np.ones(L, np.int32), np.arange(L, dtype=np.int32), table,
              0.02, 0.02, okc, ovc)
    assert np.array_equal(pool_bits(kc), okc)
    ref = pa.decode_attention(W.bits_u16(q.cpu()), okc, ovc, pa.KV_FP8_E4M3, 0.02, 0.02, table, np.array([L, L]),
                              1.0 / np.sqrt(d), flags=np.array([1, 0], np.uint8))
    got = W.bits_u16(out[1].cpu())
    from parity import compare_outputs
    compare_outputs(got[None], ref[1:2], np.array([0], np.uint8))


def test_corrupt_free_stack_and_bad_counts(gpu_device):
    # A corrupt free stack hands out ids outside [0, num_pages): page_alloc records them as they are, with
    # expected tag 0 and no tag write (every array bit-exact with the oracle), and the decode then flags
    # the sequences that use them (bit 1) and leaves their outputs untouched, tags on and off.  page_free
    # with a page count outside [0, max_pages] is status 2 and changes nothing.
    dev = gpu_device
    hkv, hq, d, ps, batch, max_pages, num_pages = 2, 8, 64, 16, 4, 6, 16
    say("corrupt free stack")
    P = Pools(dev, batch, max_pages, num_pages)
    fc = P.o["free_count"]
    # pops read entries fc-1, fc-2, ...: sequence 0 gets entries fc-1 and fc-2, sequence 1 the next three
    for idx, bad in ((fc - 2, num_pages), (fc - 4, -3), (fc - 5, -2 ** 31)):
        P.o["free_pages"][idx] = bad
        P.g["free_pages"][idx] = bad
    tags_before = P.o["tags"].copy()
    st = P.alloc([2, 3, 1, 0])
    assert st.tolist() == [0, 0, 0, 0]
    assert P.o["table"][0, 1] == num_pages and P.o["expected"][0, 1] == 0
    assert P.o["table"][1, 1] == -3 and P.o["table"][1, 2] == -2 ** 31 and P.o["expected"][1, 2] == 0
    good = [int(p) for p in P.o["table"][:3].ravel() if 0 <= p < num_pages]
    changed = np.nonzero(P.o["tags"] != tags_before)[0].tolist()
    assert sorted(changed) == sorted(good)                      # only the valid pops bumped a tag

    # decode through the pool's table: sequence 0 uses its bad slot 1, sequence 1 its slots 1-2,
    # sequence 2 only good pages, sequence 3 holds nothing (length 0)
    lens = np.array([2 * ps, 3 * ps - 5, ps, 0], np.int32)
    table = P.o["table"].copy()
    rows_k = torch.randn(batch * max_pages * ps, hkv, d, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16)
    rows_v = torch.randn(batch * max_pages * ps, hkv, d, generator=torch.Generator().manual_seed(2)).to(torch.bfloat16)
    seq = torch.arange(batch, dtype=torch.int32).repeat_interleave(max_pages * ps)
    pos = torch.arange(max_pages * ps, dtype=torch.int32).repeat(batch)
    shape = (num_pages, hkv, ps, d)
    kc = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
    vc = torch.full(shape, 0x7F, dtype=torch.uint8, device=dev)
    pt = torch.from_numpy(table).to(dev)
    fk.kv_quant_append(rows_k.to(dev), rows_v.to(dev), seq.to(dev), pos.to(dev), pt, 0.02, 0.02, kc, vc)
    okc = np.full(shape, 0x7F, np.uint8)
    ovc = np.full(shape, 0x7F, np.uint8)
    pa.append(W.bits_u16(rows_k), W.bits_u16(rows_v), seq.numpy(), pos.numpy(), table, 0.02, 0.02, okc, ovc)
    torch.cuda.synchronize()
    assert np.array_equal(pool_bits(kc), okc) and np.array_equal(pool_bits(vc), ovc)
    q = torch.randn(batch, hq, d, generator=torch.Generator().manual_seed(3)).to(torch.bfloat16)
    ws = fk.alloc_workspace(batch, hq, hkv, d, ps, max_pages, device=dev)
    for tags_on in (True, False):
        say(f"  decode through the corrupt table, tags_on={tags_on}")
        out = torch.full((batch, hq, d), 0, dtype=torch.int16, device=dev)
        out.fill_(0x7FC1)
        out = out.view(torch.bfloat16)
        flags = torch.full((batch,), 0xEE, dtype=torch.uint8, device=dev)
        ws.fill_(0xA5)
        fk.paged_decode_attn(q.to(dev), kc, vc, pt, torch.from_numpy(lens).to(dev), out, flags, ws,
                             k_scale=0.02, v_scale=0.02, page_tags=P.g["tags"] if tags_on else None,
                             expected_tags=P.g["expected"] if tags_on else None)
        torch.cuda.synchronize()
        rflags = pa.abort_flags(table, lens, ps, num_pages, P.o["tags"] if tags_on else None,
                                P.o["expected"] if tags_on else None)
        assert rflags.tolist() == [2, 2, 0, 2]
        assert np.array_equal(flags.cpu().numpy(), rflags)
        ref = pa.decode_attention(W.bits_u16(q), okc, ovc, pa.KV_FP8_E4M3, 0.02, 0.02, table, lens,
                                  1.0 / np.sqrt(d), flags=rflags)
        from parity import compare_outputs
        compare_outputs(W.bits_u16(out.cpu()), ref, rflags)

    say("bad page counts on free")
    for b, bad in ((0, -1), (1, max_pages + 1), (2, -2 ** 31)):
        P.o["counts"][b] = bad
        P.g["counts"][b] = bad
    st = P.free([1, 1, 1, 1])                                   # compares every array with the oracle
    assert st.tolist() == [pp.FREE_BAD_COUNT] * 3 + [pp.FREE_OK]
