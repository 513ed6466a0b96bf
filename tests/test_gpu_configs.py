"""Full-size workloads on the GPU, checked against the oracle on samples.

At these sizes the oracle cannot redo a whole batch quickly, so:
* abort flags are compared for every sequence (the tag rule is cheap);
* for sampled sequences, every page the GPU wrote is compared byte for byte
  with the oracle's own quantization of that sequence's rows, and every
  query head's output with the oracle's fp64 attention over those bytes;
* aborted sequences' outputs must be untouched.
The decode runs with the automatic work plan (num_blocks = 0), the launch
configuration the benchmark times.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import paged_attn as pa

from parity import (FP8_POOL_FILL, BF16_POOL_FILL, OUT_SENTINEL, bf16_bits_to_f64, compare_outputs, gpu_decode,
                    gpu_fill, pool_bits, say)

pytestmark = pytest.mark.gpu

FP8, BF16 = fk.KV_FP8_E4M3, fk.KV_BF16


def _oracle_sequence(w, b, kv_dtype):
    """The oracle's pages and outputs for sequence b alone (a one-sequence pool)."""
    L = int(w.seq_lens[b])
    n = -(-L // w.page_size)
    k, v, pos = w.rows_of(b)
    shape = (n, w.num_kv_heads, w.page_size, w.head_dim)
    if kv_dtype == FP8:
        kc, vc = np.full(shape, FP8_POOL_FILL, np.uint8), np.full(shape, FP8_POOL_FILL, np.uint8)
    else:
        kc, vc = np.full(shape, BF16_POOL_FILL, np.uint16), np.full(shape, BF16_POOL_FILL, np.uint16)
    mini_pt = np.arange(n, dtype=np.int32)[None, :]
    pa.append(W.bits_u16(k), W.bits_u16(v), np.zeros(len(pos), np.int32), pos.numpy(), mini_pt,
              w.k_scale, w.v_scale, kc, vc, kv_dtype)
    q = W.bits_u16(w.q[b:b + 1])
    out = pa.decode_attention(q, kc, vc, kv_dtype, w.k_scale, w.v_scale, mini_pt, np.array([L]),
                              w.softmax_scale, flags=np.zeros(1, np.uint8))
    return kc, vc, out[0]


def _check_config(w, kv_dtype, dev, samples, tags_on=True):
    say(f"config {w.name} kv={kv_dtype} B={w.batch} pages={w.num_pages}")
    kc, vc = gpu_fill(w, kv_dtype, dev)
    out, flags, _ = gpu_decode(w, kv_dtype, kc, vc, dev, tags_on=tags_on)
    rflags = pa.abort_flags(w.page_table, w.seq_lens, w.page_size, w.num_pages,
                            w.page_tags if tags_on else None, w.expected_tags if tags_on else None)
    assert np.array_equal(flags, rflags), f"abort flags differ at {np.nonzero(flags != rflags)[0][:10]}"
    for b in np.nonzero(flags)[0]:
        assert np.all(out[b] == OUT_SENTINEL)
    ok = [b for b in samples if flags[b] == 0]
    for b in ok:
        say(f"  sample seq {b} L={int(w.seq_lens[b])}")
        okc, ovc, ref = _oracle_sequence(w, b, kv_dtype)
        n = okc.shape[0]
        pages = torch.from_numpy(w.page_table[b, :n].astype(np.int64)).to(dev)
        assert np.array_equal(pool_bits(kc[pages]), okc), f"K pages of sequence {b} differ"
        assert np.array_equal(pool_bits(vc[pages]), ovc), f"V pages of sequence {b} differ"
        full = np.full((w.batch,) + ref.shape, np.nan)
        full[b] = ref
        sel = np.zeros((w.batch, w.num_q_heads), bool)
        sel[b] = True
        excess, rel = compare_outputs(out, full, flags, select=sel)
        raw = float(np.abs(bf16_bits_to_f64(out[b]) - ref).max())
        # one line per sampled sequence, collected into the design notes' results table
        say(f"MARGIN config={w.name} kv={'fp8' if kv_dtype == FP8 else 'bf16'} seq={b} L={int(w.seq_lens[b])} "
            f"max_abs={raw:.4e} excess_over_bf16={excess:.4e} rel_l2={rel:.4e}")
    return flags


def _samples(w, k=2):
    order = np.argsort(w.seq_lens)
    return sorted({int(order[0]), int(order[-1])} | {int(order[len(order) // 2])})[:max(k, 1) + 1]


@pytest.mark.parametrize("kv_dtype", [FP8, BF16])
def test_latency_config(gpu_device, kv_dtype):
    w = W.make("latency", device=gpu_device)
    assert _check_config(w, kv_dtype, gpu_device, [0]).tolist() == [0]


@pytest.mark.parametrize("kv_dtype", [FP8, BF16])
def test_conc32_config(gpu_device, kv_dtype):
    w = W.make("conc32", device=gpu_device)
    _check_config(w, kv_dtype, gpu_device, _samples(w))


def test_conc64_config_fp8_full_pool(gpu_device):
    w = W.make("conc64", device=gpu_device)
    flags = _check_config(w, FP8, gpu_device, _samples(w))
    assert flags.any(), "stale pages should abort some sequences"


def test_conc64_config_bf16_same_memory(gpu_device):
    w = W.make("conc64", device=gpu_device, bf16_same_memory=True)
    _check_config(w, BF16, gpu_device, _samples(w))


def test_long_config_run_a(gpu_device):
    w = W.make("long", device=gpu_device)
    assert _check_config(w, FP8, gpu_device, [3]).sum() == 0


def test_long_config_amax_scale(gpu_device):
    # the Student-t cache quantized at amax / 448: no code saturates and a few percent are subnormal
    w = W.make("long", device=gpu_device, long_scale="amax")
    assert _check_config(w, FP8, gpu_device, [5]).sum() == 0
    kc, _ = gpu_fill(w, FP8, gpu_device)            # every page of this pool is full and used
    mag = kc.view(torch.uint8) & 0x7F
    sub = float(((mag > 0) & (mag < 8)).float().mean())
    sat = float((mag == 0x7E).float().mean())
    say(f"  long amax scale: subnormal codes {100 * sub:.2f}%, saturated {100 * sat:.4f}%")
    assert 0.01 < sub < 0.10
    assert sat < 1e-4


def test_long_config_run_b_injected_mismatches(gpu_device):
    w = W.make("long", device=gpu_device, inject_tags=True)
    rflags = pa.abort_flags(w.page_table, w.seq_lens, w.page_size, w.num_pages, w.page_tags, w.expected_tags)
    assert rflags.sum() > 0, "the injection should stale some pages"
    ok = [int(b) for b in np.nonzero(rflags == 0)[0][:1]]      # may be empty: then flags only
    _check_config(w, FP8, gpu_device, ok)
