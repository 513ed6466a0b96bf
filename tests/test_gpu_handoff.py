"""Prefill -> decode hand-off on the GPU vs the oracle: amax and scale bit-exact,
and the device-scale append's cache bytes bit-exact with the oracle's append
at the oracle's scale."""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import paged_attn as pa
from oracle import scale as sc

from parity import pool_bits, say

pytestmark = pytest.mark.gpu


_WORK = {}


def _amax_gpu(x, dev):
    # one work buffer reused across calls, filled with a value above every finite bf16 before each call:
    # the result must not depend on what the buffer held
    work = _WORK.setdefault(str(dev), torch.empty(fk.AMAX_WORK_FLOATS, dtype=torch.float32, device=dev))
    work.fill_(3.0e38)
    out = torch.full((2,), -5.0, dtype=torch.float32, device=dev)
    fk.kv_absmax_scale(x.to(dev), out, work)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("n", [1, 7, 8, 9, 1000, 4096 + 3, 1 << 20, 33_554_432 + 5])
def test_absmax_scale_matches_oracle(gpu_device, n):
    say(f"absmax n={n}")
    g = torch.Generator().manual_seed(n % 1000)
    x = (torch.randn(n, generator=g) * 3.0).to(torch.bfloat16)
    if n > 8:
        x[n // 3] = float("nan"); x[n // 2] = float("inf"); x[n - 1] = -float("inf")
        x[5] = -17.25                                # the largest finite magnitude, negative
    got = _amax_gpu(x, gpu_device)
    bits = W.bits_u16(x)
    a = sc.absmax(bits)
    assert got[0] == a and got[1] == sc.scale_from_amax(a)


def test_absmax_all_bf16_patterns_and_specials(gpu_device):
    say("absmax all patterns / specials")
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    x = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16)
    got = _amax_gpu(x, gpu_device)
    assert got[0] == sc.absmax(bits) and got[1] == sc.scale_from_amax(sc.absmax(bits))
    for vals in ([0.0, -0.0], [float("nan")] * 9, [float("inf"), -float("inf")]):
        got = _amax_gpu(torch.tensor(vals).to(torch.bfloat16), gpu_device)
        assert got[0] == 0.0 and got[1] == 1.0
    assert _amax_gpu(torch.empty(0, dtype=torch.bfloat16), gpu_device).tolist() == [0.0, 1.0]


@pytest.mark.parametrize("n", [1, 9, 4096 + 3, 33_554_432 + 5])
def test_absmax_scale_pair_matches_single_calls_and_oracle(gpu_device, n):
    say(f"absmax pair n={n}")
    g = torch.Generator().manual_seed(n % 977)
    k = (torch.randn(n, generator=g) * 3.0).to(torch.bfloat16)
    v = (torch.randn(n, generator=g) * 0.5).to(torch.bfloat16)
    if n > 8:
        k[n // 3] = float("nan"); v[n // 2] = float("inf"); v[1] = -40.5
    work = torch.full((2 * fk.AMAX_WORK_FLOATS,), 3.0e38, dtype=torch.float32, device=gpu_device)
    out = torch.full((4,), -5.0, dtype=torch.float32, device=gpu_device)
    fk.kv_absmax_scale_kv(k.to(gpu_device), v.to(gpu_device), out, work)
    torch.cuda.synchronize()
    got = out.cpu().numpy()
    for t, (a_got, s_got) in ((k, got[0:2]), (v, got[2:4])):
        a = sc.absmax(W.bits_u16(t))
        assert a_got == a and s_got == sc.scale_from_amax(a)
    assert got[0:2].tolist() == _amax_gpu(k, gpu_device).tolist()
    assert got[2:4].tolist() == _amax_gpu(v, gpu_device).tolist()


def test_prefill_handoff_end_to_end(gpu_device):
    # a prefill's BF16 K/V (Student-t, so saturation and subnormals occur) -> device amax and scale ->
    # device-scale append into a permuted page pool; bytes equal the oracle's append at the oracle's scale
    say("prefill hand-off end to end")
    hkv, d, ps, L = 8, 128, 64, 4096 + 37
    w = W.make_custom([L], 64, hkv, d, ps, num_pages=-(-L // ps) + 3, seed=21, dist="t3")
    k, v, pos = w.rows_of(0)
    kd, vd = k.to(gpu_device).contiguous(), v.to(gpu_device).contiguous()
    kvs = torch.zeros(4, device=gpu_device)
    fk.kv_absmax_scale_kv(kd, vd, kvs)
    ks, vs = kvs[0:2], kvs[2:4]
    shape = (w.num_pages, hkv, ps, d)
    kc = torch.full(shape, 0x7F, dtype=torch.uint8, device=gpu_device)
    vc = torch.full(shape, 0x7F, dtype=torch.uint8, device=gpu_device)
    seq = torch.zeros(L, dtype=torch.int32, device=gpu_device)
    fk.kv_quant_append_dscale(kd, vd, seq, pos.to(gpu_device), torch.from_numpy(w.page_table).to(gpu_device),
                              ks[1:], vs[1:], kc, vc)
    torch.cuda.synchronize()
    ka, va = sc.absmax(W.bits_u16(k)), sc.absmax(W.bits_u16(v))
    k_scale, v_scale = sc.scale_from_amax(ka), sc.scale_from_amax(va)
    assert ks.cpu().numpy().tolist() == [ka, k_scale] and vs.cpu().numpy().tolist() == [va, v_scale]
    okc = np.full(shape, 0x7F, np.uint8); ovc = np.full(shape, 0x7F, np.uint8)
    pa.append(W.bits_u16(k), W.bits_u16(v), np.zeros(L, np.int32), pos.numpy(), w.page_table, float(k_scale),
              float(v_scale), okc, ovc)
    assert np.array_equal(pool_bits(kc), okc) and np.array_equal(pool_bits(vc), ovc)
    # the largest magnitude of each tensor became +-448 (code 0x7E / 0xFE)
    assert {0x7E, 0xFE} & set(np.unique(pool_bits(kc)).tolist())


def test_dscale_append_with_invalid_scale_writes_nothing(gpu_device):
    say("dscale append invalid scale")
    hkv, d, ps = 2, 64, 16
    kc = torch.full((4, hkv, ps, d), 0x33, dtype=torch.uint8, device=gpu_device)
    vc = kc.clone()
    rows = torch.ones(3, hkv, d, dtype=torch.bfloat16, device=gpu_device)
    pt = torch.tensor([[0, 1, 2, 3]], dtype=torch.int32, device=gpu_device)
    for bad in (0.0, -1.0, float("nan"), float("inf")):
        s = torch.tensor([bad], dtype=torch.float32, device=gpu_device)
        good = torch.tensor([1.0], dtype=torch.float32, device=gpu_device)
        fk.kv_quant_append_dscale(rows, rows, torch.zeros(3, dtype=torch.int32, device=gpu_device),
                                  torch.arange(3, dtype=torch.int32, device=gpu_device), pt, s, good, kc, vc)
    torch.cuda.synchronize()
    assert int((kc != 0x33).sum()) == 0 and int((vc != 0x33).sum()) == 0
