"""kv_quant_append on the GPU vs the oracle: cache bytes bit-exact.

Every one of the 65,536 BF16 bit patterns (NaNs, infinities, subnormals,
signed zeros included) is quantized with several scales and scattered through
a permuted page table into a pool pre-filled with a sentinel; the whole pool
(written and unwritten bytes) must equal the oracle's.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import paged_attn as pa

from parity import pool_bits, say

pytestmark = pytest.mark.gpu


def _all_bf16_rows(hkv, d):
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    rows = bits.reshape(-1, hkv, d)
    return torch.from_numpy(rows.view(np.int16)).view(torch.bfloat16), rows


def _layout(n_rows, page_size, batch, seed):
    per_seq = n_rows // batch
    pages_per_seq = -(-per_seq // page_size)
    pool = batch * pages_per_seq + 5
    perm = np.random.default_rng(seed).permutation(pool)
    pt = perm[:batch * pages_per_seq].reshape(batch, pages_per_seq).astype(np.int32)
    seq = np.repeat(np.arange(batch), per_seq).astype(np.int32)
    pos = np.tile(np.arange(per_seq), batch).astype(np.int32)
    return pt, seq, pos, pool


@pytest.mark.parametrize("scale", [1.0, 0.0288, 3.57, 2.0 ** -3, 1.2e-5, 7.5e35])
@pytest.mark.parametrize("hkv,d,ps", [(2, 64, 16), (8, 128, 64), (4, 128, 256)])
def test_append_fp8_all_bf16_patterns(gpu_device, scale, hkv, d, ps):
    say(f"append fp8 all-bf16 scale={scale} hkv={hkv} d={d} ps={ps}")
    t, rows = _all_bf16_rows(hkv, d)
    n = rows.shape[0]
    pt, seq, pos, pool = _layout(n, ps, 4, seed=int(scale * 1000) % 97 + d)
    shape = (pool, hkv, ps, d)
    kc = torch.full(shape, 0xA5, dtype=torch.uint8, device=gpu_device)
    vc = torch.full(shape, 0x5A, dtype=torch.uint8, device=gpu_device)
    # V gets the patterns in reverse so K and V rows differ
    vt = torch.flip(t.view(-1), [0]).view(t.shape).contiguous()
    fk.kv_quant_append(t.to(gpu_device), vt.to(gpu_device), torch.from_numpy(seq).to(gpu_device),
                       torch.from_numpy(pos).to(gpu_device), torch.from_numpy(pt).to(gpu_device),
                       scale, scale * 0.5, kc, vc, fk.KV_FP8_E4M3)
    torch.cuda.synchronize()
    okc = np.full(shape, 0xA5, np.uint8)
    ovc = np.full(shape, 0x5A, np.uint8)
    pa.append(rows, W.bits_u16(vt), seq, pos, pt, scale, scale * 0.5, okc, ovc, pa.KV_FP8_E4M3)
    gk, gv = pool_bits(kc), pool_bits(vc)
    bad = np.nonzero(gk.ravel() != okc.ravel())[0]
    assert bad.size == 0, f"{bad.size} K bytes differ, first at {bad[:5]}"
    assert np.array_equal(gv, ovc)


def _many_scales():
    """Scales that stress the multiply-and-correct quotient: subnormal and
    near-overflow scales, scales whose reciprocal is inexact, and 16 seeded
    log-uniform ones."""
    fixed = [3 * 2.0 ** -149, 1e-40, 2.0 ** -126, 1e-30, 3.3e-9, 2.0 ** -10, 0.3, 1.0000001, 1.7, 3.0,
             448.0, 1e10, 3.0e38]
    rng = np.random.default_rng(11)
    return fixed + [float(np.float32(2.0 ** e)) for e in rng.uniform(-120, 120, 16)]


@pytest.mark.parametrize("scale", _many_scales())
def test_append_fp8_all_bf16_patterns_many_scales(gpu_device, scale):
    say(f"append fp8 all-bf16 scale={scale!r} (many scales)")
    hkv, d, ps = 8, 128, 64
    t, rows = _all_bf16_rows(hkv, d)
    n = rows.shape[0]
    pt, seq, pos, pool = _layout(n, ps, 2, seed=7)
    shape = (pool, hkv, ps, d)
    kc = torch.full(shape, 0xA5, dtype=torch.uint8, device=gpu_device)
    vc = torch.full(shape, 0x5A, dtype=torch.uint8, device=gpu_device)
    vt = torch.flip(t.view(-1), [0]).view(t.shape).contiguous()
    v_scale = float(np.float32(min(scale * 1.37, 3.0e38)))
    fk.kv_quant_append(t.to(gpu_device), vt.to(gpu_device), torch.from_numpy(seq).to(gpu_device),
                       torch.from_numpy(pos).to(gpu_device), torch.from_numpy(pt).to(gpu_device),
                       scale, v_scale, kc, vc, fk.KV_FP8_E4M3)
    torch.cuda.synchronize()
    okc = np.full(shape, 0xA5, np.uint8)
    ovc = np.full(shape, 0x5A, np.uint8)
    pa.append(rows, W.bits_u16(vt), seq, pos, pt, scale, v_scale, okc, ovc, pa.KV_FP8_E4M3)
    gk, gv = pool_bits(kc), pool_bits(vc)
    bad = np.nonzero(gk.ravel() != okc.ravel())[0]
    assert bad.size == 0, f"{bad.size} K bytes differ, first at {bad[:5]}"
    badv = np.nonzero(gv.ravel() != ovc.ravel())[0]
    assert badv.size == 0, f"{badv.size} V bytes differ, first at {badv[:5]}"


@pytest.mark.parametrize("hkv,d,ps", [(2, 64, 16), (8, 128, 64)])
def test_append_bf16_copies_bits(gpu_device, hkv, d, ps):
    say(f"append bf16 copy all patterns hkv={hkv} d={d} ps={ps}")
    t, rows = _all_bf16_rows(hkv, d)
    vrows = np.ascontiguousarray(rows[::-1, :, ::-1])     # V: the same patterns in another order
    tv = torch.from_numpy(vrows.view(np.int16)).view(torch.bfloat16)
    pt, seq, pos, pool = _layout(rows.shape[0], ps, 4, seed=3)
    shape = (pool, hkv, ps, d)
    fill = torch.tensor(0x1234, dtype=torch.int16).view(torch.bfloat16).item()
    kc = torch.full(shape, fill, dtype=torch.bfloat16, device=gpu_device)
    vc = torch.full(shape, fill, dtype=torch.bfloat16, device=gpu_device)
    fk.kv_quant_append(t.to(gpu_device), tv.to(gpu_device), torch.from_numpy(seq).to(gpu_device),
                       torch.from_numpy(pos).to(gpu_device), torch.from_numpy(pt).to(gpu_device),
                       1.0, 1.0, kc, vc, fk.KV_BF16)
    torch.cuda.synchronize()
    okc = np.full(shape, 0x1234, np.uint16)
    ovc = np.full(shape, 0x1234, np.uint16)
    pa.append(rows, vrows, seq, pos, pt, 1.0, 1.0, okc, ovc, pa.KV_BF16)
    assert np.array_equal(pool_bits(kc), okc) and np.array_equal(pool_bits(vc), ovc)


@pytest.mark.parametrize("kv_dtype", [fk.KV_FP8_E4M3, fk.KV_BF16])
def test_append_skips_rows_without_a_valid_destination(gpu_device, kv_dtype):
    say(f"append skip rules kv_dtype={kv_dtype}")
    hkv, d, ps, pool = 2, 64, 16, 6
    pt = np.array([[1, -1, 3], [7, 0, 2]], np.int32)          # page 7 is outside a 6-page pool
    seq = np.array([0, 0, 1, 1, 2, -1, 0, 1, 0], np.int32)
    pos = np.array([3, 20, 5, 17, 0, 0, 48, 40, -1], np.int32)  # only rows 0 and 3 and 7 land
    rng = np.random.default_rng(0)
    x = torch.from_numpy(rng.standard_normal((9, hkv, d)).astype(np.float32)).to(torch.bfloat16)
    dt = torch.uint8 if kv_dtype == fk.KV_FP8_E4M3 else torch.bfloat16
    kc = torch.zeros((pool, hkv, ps, d), dtype=dt, device=gpu_device)
    vc = torch.zeros((pool, hkv, ps, d), dtype=dt, device=gpu_device)
    fk.kv_quant_append(x.to(gpu_device), x.to(gpu_device), torch.from_numpy(seq).to(gpu_device),
                       torch.from_numpy(pos).to(gpu_device), torch.from_numpy(pt).to(gpu_device),
                       0.01, 0.02, kc, vc, kv_dtype)
    torch.cuda.synchronize()
    npdt = np.uint8 if kv_dtype == fk.KV_FP8_E4M3 else np.uint16
    okc = np.zeros((pool, hkv, ps, d), npdt)
    ovc = np.zeros((pool, hkv, ps, d), npdt)
    n = pa.append(W.bits_u16(x), W.bits_u16(x), seq, pos, pt, 0.01, 0.02, okc, ovc, kv_dtype)
    assert n == 3
    assert np.array_equal(pool_bits(kc), okc) and np.array_equal(pool_bits(vc), ovc)
