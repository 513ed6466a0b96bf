"""Shared harness for GPU-vs-oracle parity tests (imported by tests, not collected).

The HIP path and the oracle receive the same seeded inputs from
``decode_attention_fp8_kv_amd.workloads``.  Each side fills its own cache
(HIP: ``kv_quant_append`` on the GPU; oracle: ``oracle.paged_attn.append`` in
numpy), runs its own attention, and the results are compared:

* cache bytes and abort flags: bit-exact;
* outputs of non-aborted sequences: max |gpu - oracle| <= 2e-2 beyond the
  output's own BF16 rounding (|bf16(oracle) - oracle|), and relative L2
  error <= 5e-3 over all compared elements;
* outputs of aborted sequences: left exactly as they were (a sentinel).
"""

from __future__ import annotations

import sys

import numpy as np
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import e4m3
from oracle import paged_attn as pa

ATOL = 2e-2
REL_L2 = 5e-3
OUT_SENTINEL = 0x7FC1          # a BF16 NaN pattern nobody writes
FP8_POOL_FILL = 0x7F           # e4m3 NaN code in every slot not appended
BF16_POOL_FILL = 0x7FC0        # BF16 NaN in every slot not appended


def say(msg: str) -> None:
    """Name the case before any GPU step, so a crash log points at it."""
    print(msg, flush=True)
    sys.stdout.flush()


def _np_pool(w, kv_dtype):
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    if kv_dtype == W.KV_FP8_E4M3:
        return np.full(shape, FP8_POOL_FILL, np.uint8), np.full(shape, FP8_POOL_FILL, np.uint8)
    return np.full(shape, BF16_POOL_FILL, np.uint16), np.full(shape, BF16_POOL_FILL, np.uint16)


def _gpu_pool(w, kv_dtype, dev):
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    if kv_dtype == W.KV_FP8_E4M3:
        return (torch.full(shape, FP8_POOL_FILL, dtype=torch.uint8, device=dev),
                torch.full(shape, FP8_POOL_FILL, dtype=torch.uint8, device=dev))
    fill = torch.tensor(BF16_POOL_FILL, dtype=torch.int16).view(torch.bfloat16).item()
    return (torch.full(shape, fill, dtype=torch.bfloat16, device=dev),
            torch.full(shape, fill, dtype=torch.bfloat16, device=dev))


def pool_bits(t: torch.Tensor) -> np.ndarray:
    if t.dtype == torch.bfloat16:
        return W.bits_u16(t)
    return t.cpu().numpy()


def gpu_fill(w, kv_dtype, dev, include_new=True):
    """Caches filled on the GPU by kv_quant_append (context rows, then the step's new rows)."""
    kc, vc = _gpu_pool(w, kv_dtype, dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    fk.kv_quant_append(w.ctx_k.to(dev).contiguous(), w.ctx_v.to(dev).contiguous(), w.ctx_seq.to(dev),
                       w.ctx_pos.to(dev), pt, w.k_scale, w.v_scale, kc, vc, kv_dtype)
    if include_new and w.new_k.shape[0]:
        fk.kv_quant_append(w.new_k.to(dev).contiguous(), w.new_v.to(dev).contiguous(), w.new_seq.to(dev),
                           w.new_pos.to(dev), pt, w.k_scale, w.v_scale, kc, vc, kv_dtype)
    return kc, vc


def oracle_fill(w, kv_dtype, include_new=True):
    kc, vc = _np_pool(w, kv_dtype)
    pa.append(W.bits_u16(w.ctx_k), W.bits_u16(w.ctx_v), w.ctx_seq.cpu().numpy(), w.ctx_pos.cpu().numpy(),
              w.page_table, w.k_scale, w.v_scale, kc, vc, kv_dtype)
    if include_new and w.new_k.shape[0]:
        pa.append(W.bits_u16(w.new_k), W.bits_u16(w.new_v), w.new_seq.cpu().numpy(), w.new_pos.cpu().numpy(),
                  w.page_table, w.k_scale, w.v_scale, kc, vc, kv_dtype)
    return kc, vc


def gpu_decode(w, kv_dtype, kc, vc, dev, tags_on=True, num_blocks=0, seq_lens=None, page_table=None,
               page_tags=None, expected_tags=None):
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    page_table = w.page_table if page_table is None else page_table
    page_tags = w.page_tags if page_tags is None else page_tags
    expected_tags = w.expected_tags if expected_tags is None else expected_tags
    out = torch.full(tuple(w.q.shape), 0, dtype=torch.int16, device=dev)
    out.fill_(OUT_SENTINEL)
    out = out.view(torch.bfloat16)
    flags = torch.full((w.batch,), 0xEE, dtype=torch.uint8, device=dev)
    ws = fk.alloc_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                            page_table.shape[1], num_blocks, device=dev)
    ws.fill_(0xA5)  # the workspace needs no initialization: start from garbage
    tags = torch.from_numpy(page_tags.view(np.int32)).to(dev) if tags_on else None
    exp = torch.from_numpy(np.ascontiguousarray(expected_tags).view(np.int32)).to(dev) if tags_on else None
    fk.paged_decode_attn(w.q.to(dev).contiguous(), kc, vc, torch.from_numpy(page_table).to(dev),
                         torch.from_numpy(np.asarray(seq_lens, np.int32)).to(dev), out, flags, ws,
                         kv_dtype=kv_dtype, k_scale=w.k_scale, v_scale=w.v_scale, page_tags=tags,
                         expected_tags=exp, softmax_scale=w.softmax_scale, num_blocks=num_blocks)
    torch.cuda.synchronize(dev)
    return W.bits_u16(out), flags.cpu().numpy(), ws


def oracle_decode(w, kv_dtype, kc, vc, tags_on=True, seq_lens=None, page_table=None, page_tags=None,
                  expected_tags=None, batch_indices=None, q_heads=None):
    seq_lens = w.seq_lens if seq_lens is None else seq_lens
    page_table = w.page_table if page_table is None else page_table
    page_tags = w.page_tags if page_tags is None else page_tags
    expected_tags = w.expected_tags if expected_tags is None else expected_tags
    flags = pa.abort_flags(page_table, seq_lens, w.page_size, w.num_pages,
                           page_tags if tags_on else None, expected_tags if tags_on else None)
    out = pa.decode_attention(W.bits_u16(w.q), kc, vc, kv_dtype, w.k_scale, w.v_scale, page_table,
                              seq_lens, w.softmax_scale, flags=flags, batch_indices=batch_indices,
                              q_heads=q_heads)
    return out, flags


def bf16_bits_to_f64(bits: np.ndarray) -> np.ndarray:
    return e4m3.bf16_bits_to_f32(bits).astype(np.float64)


def _bf16_round(x: np.ndarray) -> np.ndarray:
    return torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).to(torch.float64).numpy()


def compare_outputs(gpu_bits, ref, flags, select=None):
    """Check GPU outputs against the fp64 oracle; returns (max_abs_excess, rel_l2).

    ``select``: boolean mask [B][Hq] of the (sequence, head) rows to compare
    (default: every row of every non-aborted sequence).
    """
    B, Hq, _ = ref.shape
    ok_rows = np.repeat((np.asarray(flags) == 0)[:, None], Hq, axis=1)
    sel = ok_rows if select is None else (ok_rows & select)
    got = bf16_bits_to_f64(gpu_bits)[sel]
    want = ref[sel]
    assert np.isfinite(want).all(), "oracle produced non-finite values for a compared row"
    assert np.isfinite(got).all(), "GPU produced non-finite values"
    err = np.abs(got - want)
    floor = np.abs(_bf16_round(want) - want)
    excess = float((err - floor).max()) if err.size else 0.0
    rel = float(np.linalg.norm(got - want) / max(np.linalg.norm(want), 1e-30)) if err.size else 0.0
    raw = float(err.max()) if err.size else 0.0
    say(f"  margins: max|gpu-oracle| {raw:.3e}, beyond bf16 rounding {excess:.3e} (limit 2e-2), "
        f"bf16 floor {float(floor.max()) if err.size else 0.0:.3e}, rel-L2 {rel:.3e} (limit 5e-3), "
        f"|oracle| max {float(np.abs(want).max()) if err.size else 0.0:.3g}")
    assert excess <= ATOL, f"max |gpu - oracle| exceeds 2e-2 beyond bf16 rounding: {excess:.3g}"
    assert rel <= REL_L2, f"relative L2 error {rel:.3g} > 5e-3"
    # aborted sequences: untouched
    for b in np.nonzero(np.asarray(flags) != 0)[0]:
        assert np.all(gpu_bits[b] == OUT_SENTINEL), f"output of aborted sequence {b} was written"
    return excess, rel
