"""Pins for the oracle's append, tag rule and fp64 paged attention (CPU only).

Pinned against: hand-worked layout examples, closed forms of softmax
attention (one token, equal keys -> mean of V, two tokens -> logistic
weights, a dominant key), invariances (physical page permutation, softmax
scale), the query-head -> KV-head grouping, torch's fp64
``scaled_dot_product_attention`` on the logical (unpaged) rows, a brute-force
per-element evaluation on tiny inputs, and the tag rule's truth table as the
pages state it in prose.
"""

import math
import os

import numpy as np
import pytest
import torch

from oracle import e4m3
from oracle import paged_attn as pa

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _bf16(x):
    """float -> BF16 bits via torch's round-to-nearest-even cast."""
    t = torch.as_tensor(np.asarray(x, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def _f(bits):
    return e4m3.bf16_bits_to_f32(bits).astype(np.float64)


def _build(lengths, hkv, d, ps, pool, rng, kv_dtype=pa.KV_FP8_E4M3, perm=None,
           k_rows=None, v_rows=None):
    """Random logical K/V rows, a permuted page table, and the oracle-filled caches."""
    b = len(lengths)
    max_pages = max(-(-L // ps) for L in lengths)
    need = sum(-(-L // ps) for L in lengths)
    perm = rng.permutation(pool)[:need] if perm is None else perm
    pt = np.full((b, max_pages), -1, np.int32)
    k_rows = k_rows or [_bf16(rng.standard_normal((L, hkv, d))) for L in lengths]
    v_rows = v_rows or [_bf16(rng.standard_normal((L, hkv, d))) for L in lengths]
    i = 0
    for s, L in enumerate(lengths):
        n = -(-L // ps)
        pt[s, :n] = perm[i:i + n]
        i += n
    dt = np.uint8 if kv_dtype == pa.KV_FP8_E4M3 else np.uint16
    fill = 0x7F if kv_dtype == pa.KV_FP8_E4M3 else 0x7FC0      # NaN everywhere unwritten
    kc = np.full((pool, hkv, ps, d), fill, dt)
    vc = np.full((pool, hkv, ps, d), fill, dt)
    amax_k = max(np.abs(_f(r)).max() for r in k_rows)
    amax_v = max(np.abs(_f(r)).max() for r in v_rows)
    ks, vs = np.float32(amax_k / 448.0), np.float32(amax_v / 448.0)
    for s, L in enumerate(lengths):
        pa.append(k_rows[s], v_rows[s], np.full(L, s), np.arange(L), pt, ks, vs, kc, vc, kv_dtype)
    return dict(pt=pt, kc=kc, vc=vc, ks=ks, vs=vs, k_rows=k_rows, v_rows=v_rows)


# ---------------------------------------------------------------- append ----
def test_append_layout_hand_example():
    # 2 sequences, page size 2, 1 KV head, head_dim 1, pool of 4 pages.
    pt = np.array([[3, 0], [2, -1]], np.int32)
    kc = np.zeros((4, 1, 2, 1), np.uint16)
    vc = np.zeros((4, 1, 2, 1), np.uint16)
    rows = np.arange(1, 6, dtype=np.uint16).reshape(5, 1, 1)          # K bits 1..5
    seq = np.array([0, 0, 0, 1, 1])
    pos = np.array([0, 1, 2, 0, 1])
    n = pa.append(rows, rows + 100, seq, pos, pt, 1.0, 1.0, kc, vc, pa.KV_BF16)
    assert n == 5
    # seq 0 tokens 0,1 -> page 3 slots 0,1; token 2 -> page 0 slot 0; seq 1 -> page 2
    assert kc[3, 0, :, 0].tolist() == [1, 2]
    assert kc[0, 0, :, 0].tolist() == [3, 0]
    assert kc[2, 0, :, 0].tolist() == [4, 5]
    assert vc[2, 0, :, 0].tolist() == [104, 105]
    assert kc[1].sum() == 0


def test_append_head_major_layout():
    # cache[page][head][slot][d]: one row with 2 heads x 3 dims into slot 1 of page 0
    pt = np.array([[0]], np.int32)
    kc = np.zeros((1, 2, 2, 3), np.uint16)
    vc = np.zeros((1, 2, 2, 3), np.uint16)
    row = np.array([[[1, 2, 3], [4, 5, 6]]], np.uint16)
    pa.append(row, row, [0], [1], pt, 1.0, 1.0, kc, vc, pa.KV_BF16)
    assert kc[0, 0, 1].tolist() == [1, 2, 3] and kc[0, 1, 1].tolist() == [4, 5, 6]
    assert kc[0, :, 0].sum() == 0


def test_append_skips_out_of_range_rows():
    pt = np.array([[1, -1], [5, 0]], np.int32)      # page 5 is outside a 2-page pool
    kc = np.full((2, 1, 2, 2), 0xAA, np.uint8)
    vc = np.full((2, 1, 2, 2), 0xAA, np.uint8)
    rows = _bf16(np.ones((6, 1, 2)))
    seq = np.array([0, 0, 1, 2, -1, 1])
    pos = np.array([0, 2, 0, 0, 0, 4])               # pos 2 -> table entry -1; 4 >= 2*2
    n = pa.append(rows, rows, seq, pos, pt, 1.0, 1.0, kc, vc)
    assert n == 1                                    # only (seq 0, pos 0) -> page 1 slot 0
    assert kc[1, 0, 0].tolist() == [0x38, 0x38]      # 1.0 -> 0x38
    untouched = np.ones_like(kc, bool)
    untouched[1, 0, 0] = False
    assert np.all(kc[untouched] == 0xAA) and np.all(vc[untouched] == 0xAA)


def test_append_quantizes_k_and_v_with_their_own_scales():
    pt = np.array([[0]], np.int32)
    kc = np.zeros((1, 1, 1, 1), np.uint8)
    vc = np.zeros((1, 1, 1, 1), np.uint8)
    pa.append(_bf16([[[3.0]]]), _bf16([[[3.0]]]), [0], [0], pt, 2.0, 0.5, kc, vc)
    assert e4m3.decode(kc[0, 0, 0, 0]) == 1.5 and e4m3.decode(vc[0, 0, 0, 0]) == 6.0


# ------------------------------------------------------------------ tags ----
def _flags(pt, lens, ps, num_pages, tags=None, exp=None):
    return pa.abort_flags(np.array(pt), np.array(lens), ps, num_pages,
                          None if tags is None else np.array(tags, np.uint32),
                          None if exp is None else np.array(exp, np.uint32)).tolist()


def test_tag_rule_truth_table():
    ps, P = 4, 8
    tags = [10, 11, 12, 13, 14, 15, 16, 17]
    pt = [[2, 5, 7, -1]]
    good = [[12, 15, 17, 0]]
    # all pages used by the sequence match -> no abort; with or without tags
    assert _flags(pt, [9], ps, P, tags, good) == [0]
    assert _flags(pt, [9], ps, P) == [0]
    # a mismatch in a fully used page -> bit 0
    assert _flags(pt, [9], ps, P, tags, [[12, 99, 17, 0]]) == [1]
    # a mismatch in the partial last page (token 8 lives in slot 2) -> bit 0
    assert _flags(pt, [9], ps, P, tags, [[12, 15, 99, 0]]) == [1]
    # ... but with length 8 slot 2 is not read, so its tag is not checked
    assert _flags(pt, [8], ps, P, tags, [[12, 15, 99, 0]]) == [0]
    # tags off: mismatching expected values are ignored
    assert _flags(pt, [9], ps, P, None, None) == [0]
    # page id out of range among the used pages -> bit 1 (tag never compared)
    assert _flags([[2, 9, 7, -1]], [9], ps, P, tags, good) == [2]
    assert _flags([[2, -3, 7, -1]], [9], ps, P, tags, good) == [2]
    # both conditions at once
    assert _flags([[2, 9, 7, -1]], [9], ps, P, tags, [[99, 0, 17, 0]]) == [3]
    # unusable lengths -> bit 1
    assert _flags(pt, [0], ps, P, tags, good) == [2]
    assert _flags(pt, [17], ps, P, tags, good) == [2]
    assert _flags(pt, [16], ps, P, None, None) == [2]     # page -1 in slot 3
    # per sequence: only the sequence that saw the stale page aborts
    assert _flags([[2, -1], [3, 4]], [3, 5], ps, P, tags,
                  [[12, 0], [13, 0]]) == [0, 1]


def test_stale_page_after_reallocation_aborts():
    # A page reallocated to someone else gets a new generation; the old owner
    # still expects the old one and must abort rather than read it.
    ps, P = 2, 4
    tags = np.array([7, 7, 7, 7], np.uint32)
    pt = np.array([[0, 1], [2, 3]], np.int32)
    exp = np.array([[7, 7], [7, 7]], np.uint32)
    assert _flags(pt, [4, 4], ps, P, tags, exp) == [0, 0]
    tags[1] += 1                                       # page 1 reallocated
    assert _flags(pt, [4, 4], ps, P, tags, exp) == [1, 0]


# ------------------------------------------------------------- attention ----
def test_single_token_returns_its_value_row():
    rng = np.random.default_rng(1)
    w = _build([1], 2, 16, 4, 4, rng)
    q = _bf16(rng.standard_normal((1, 4, 16)))
    out = pa.decode_attention(q, w["kc"], w["vc"], pa.KV_FP8_E4M3, w["ks"], w["vs"],
                              w["pt"], [1], 0.25)
    v0 = e4m3.dequantize(e4m3.quantize(w["v_rows"][0][0], w["vs"]), w["vs"])  # [hkv][d]
    assert np.array_equal(out[0], v0[[0, 0, 1, 1]])


def test_equal_keys_give_mean_of_values():
    rng = np.random.default_rng(2)
    L, hkv, d = 37, 2, 8
    k_rows = [np.repeat(_bf16(rng.standard_normal((1, hkv, d))), L, axis=0)]
    w = _build([L], hkv, d, 8, 10, rng, k_rows=k_rows)
    q = _bf16(rng.standard_normal((1, 2 * hkv, d)))
    out = pa.decode_attention(q, w["kc"], w["vc"], pa.KV_FP8_E4M3, w["ks"], w["vs"],
                              w["pt"], [L], 0.3)
    vdq = e4m3.dequantize(e4m3.quantize(w["v_rows"][0], w["vs"]), w["vs"])   # [L][hkv][d]
    mean = vdq.mean(axis=0)
    np.testing.assert_allclose(out[0], mean[[0, 0, 1, 1]], rtol=0, atol=1e-13)


def test_two_tokens_logistic_weights():
    # q.k0 - q.k1 = delta  ->  weights sigmoid(+-softmax_scale*delta)
    d = 4
    q = _bf16([[[1.0, 0.0, 0.0, 0.0]]])
    k_rows = [_bf16([[[2.0, 1, 1, 1]], [[0.5, 1, 1, 1]]])]
    v_rows = [_bf16([[[1.0, 2, 3, 4]], [[-1.0, 0, 5, 8]]])]
    w = _build([2], 1, d, 2, 1, np.random.default_rng(0), kv_dtype=pa.KV_BF16,
               k_rows=k_rows, v_rows=v_rows)
    scale = 0.75
    out = pa.decode_attention(q, w["kc"], w["vc"], pa.KV_BF16, 1.0, 1.0, w["pt"], [2], scale)
    a = 1.0 / (1.0 + math.exp(-scale * (2.0 - 0.5)))
    expect = a * np.array([1.0, 2, 3, 4]) + (1 - a) * np.array([-1.0, 0, 5, 8])
    np.testing.assert_allclose(out[0, 0], expect, rtol=1e-14, atol=1e-14)


def test_dominant_key_selects_its_value():
    rng = np.random.default_rng(4)
    L, d = 50, 8
    k = rng.standard_normal((L, 1, d)) * 0.01
    k[17, 0, :] = 40.0
    w = _build([L], 1, d, 16, 4, rng, kv_dtype=pa.KV_BF16, k_rows=[_bf16(k)])
    q = _bf16(np.full((1, 1, d), 1.0))
    out = pa.decode_attention(q, w["kc"], w["vc"], pa.KV_BF16, 1, 1, w["pt"], [L], 1.0)
    np.testing.assert_allclose(out[0, 0], _f(w["v_rows"][0][17, 0]), rtol=0, atol=1e-12)


def test_query_heads_read_their_group_kv_head():
    # V of KV head g is the constant g+1 -> every query head in group g outputs g+1.
    rng = np.random.default_rng(5)
    L, hkv, d, grp = 20, 4, 8, 3
    v = np.ones((L, hkv, d)) * (np.arange(hkv)[None, :, None] + 1.0)
    w = _build([L], hkv, d, 4, 8, rng, kv_dtype=pa.KV_BF16, v_rows=[_bf16(v)])
    q = _bf16(rng.standard_normal((1, hkv * grp, d)))
    out = pa.decode_attention(q, w["kc"], w["vc"], pa.KV_BF16, 1, 1, w["pt"], [L], 0.2)
    for h in range(hkv * grp):
        np.testing.assert_allclose(out[0, h], h // grp + 1.0, rtol=1e-14)


def test_physical_page_permutation_is_invisible():
    rng = np.random.default_rng(6)
    lengths, hkv, d, ps = [45, 13], 2, 16, 8
    base = _build(lengths, hkv, d, ps, 12, rng)
    q = _bf16(rng.standard_normal((2, 4, d)))
    outs = []
    for seed in range(3):
        w = _build(lengths, hkv, d, ps, 12 + seed, np.random.default_rng(100 + seed),
                   k_rows=base["k_rows"], v_rows=base["v_rows"])
        outs.append(pa.decode_attention(q, w["kc"], w["vc"], pa.KV_FP8_E4M3, w["ks"], w["vs"],
                                        w["pt"], lengths, 0.25))
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])


def test_softmax_scale_trades_with_query_scale():
    rng = np.random.default_rng(8)
    w = _build([30], 1, 8, 8, 4, rng)
    q = rng.standard_normal((1, 2, 8))
    a = pa.decode_attention(_bf16(q), w["kc"], w["vc"], 0, w["ks"], w["vs"], w["pt"], [30], 0.5)
    b = pa.decode_attention(_bf16(2 * q), w["kc"], w["vc"], 0, w["ks"], w["vs"], w["pt"], [30], 0.25)
    np.testing.assert_allclose(a, b, rtol=1e-13, atol=1e-13)


@pytest.mark.parametrize("kv_dtype", [pa.KV_FP8_E4M3, pa.KV_BF16])
def test_matches_torch_sdpa_on_logical_rows(kv_dtype):
    # The paged, permuted, possibly quantized cache must attend exactly like
    # torch's fp64 SDPA over the logical rows (dequantized the same way).
    rng = np.random.default_rng(9)
    lengths, hkv, grp, d, ps = [100, 257, 16], 2, 4, 64, 16
    w = _build(lengths, hkv, d, ps, 64, rng, kv_dtype=kv_dtype)
    q = _bf16(rng.standard_normal((3, hkv * grp, d)))
    sm = 0.125
    out = pa.decode_attention(q, w["kc"], w["vc"], kv_dtype, w["ks"], w["vs"], w["pt"],
                              lengths, sm)
    for b, L in enumerate(lengths):
        if kv_dtype == pa.KV_FP8_E4M3:
            K = e4m3.dequantize(e4m3.quantize(w["k_rows"][b], w["ks"]), w["ks"])
            V = e4m3.dequantize(e4m3.quantize(w["v_rows"][b], w["vs"]), w["vs"])
        else:
            K, V = _f(w["k_rows"][b]), _f(w["v_rows"][b])
        Kt = torch.from_numpy(K).permute(1, 0, 2).repeat_interleave(grp, 0)   # [Hq][L][D]
        Vt = torch.from_numpy(V).permute(1, 0, 2).repeat_interleave(grp, 0)
        Qt = torch.from_numpy(_f(q[b]))[:, None, :]                            # [Hq][1][D]
        ref = torch.nn.functional.scaled_dot_product_attention(Qt, Kt, Vt, scale=sm)[:, 0, :]
        np.testing.assert_allclose(out[b], ref.numpy(), rtol=1e-12, atol=1e-12)


def test_brute_force_per_element_tiny():
    # Token-by-token page walk with math.exp / math.fsum, no numpy algebra.
    rng = np.random.default_rng(10)
    lengths, hkv, grp, d, ps = [5, 3], 2, 2, 4, 2
    w = _build(lengths, hkv, d, ps, 6, rng)
    q = _bf16(rng.standard_normal((2, hkv * grp, d)))
    sm = float(np.float32(0.7))
    out = pa.decode_attention(q, w["kc"], w["vc"], 0, w["ks"], w["vs"], w["pt"], lengths, sm)
    lut = e4m3.decode_lut()
    for b, L in enumerate(lengths):
        for h in range(hkv * grp):
            g = h // grp
            qv = [float(x) for x in _f(q[b, h])]
            keys, vals = [], []
            for t in range(L):
                page, slot = int(w["pt"][b][t // ps]), t % ps
                keys.append([lut[w["kc"][page, g, slot, i]] * float(w["ks"]) for i in range(d)])
                vals.append([lut[w["vc"][page, g, slot, i]] * float(w["vs"]) for i in range(d)])
            s = [sm * math.fsum(qv[i] * keys[t][i] for i in range(d)) for t in range(L)]
            mx = max(s)
            e = [math.exp(x - mx) for x in s]
            z = math.fsum(e)
            for i in range(d):
                o = math.fsum(e[t] * vals[t][i] for t in range(L)) / z
                assert abs(o - out[b, h, i]) <= 1e-12 * max(1.0, abs(o))


def test_unwritten_slots_and_pages_are_never_read():
    # _build fills every unwritten byte with the NaN code; outputs stay finite,
    # and table entries past the used pages are -1 (would fault if gathered).
    rng = np.random.default_rng(11)
    lengths = [17, 1, 64]
    w = _build(lengths, 2, 8, 16, 16, rng)
    assert (w["pt"] == -1).any()
    q = _bf16(rng.standard_normal((3, 2, 8)))
    out = pa.decode_attention(q, w["kc"], w["vc"], 0, w["ks"], w["vs"], w["pt"], lengths, 0.3)
    assert np.isfinite(out).all()


def test_aborted_sequences_get_no_output():
    rng = np.random.default_rng(12)
    w = _build([10, 10], 1, 8, 4, 8, rng)
    q = _bf16(rng.standard_normal((2, 1, 8)))
    flags = np.array([0, 1], np.uint8)
    out = pa.decode_attention(q, w["kc"], w["vc"], 0, w["ks"], w["vs"], w["pt"], [10, 10],
                              0.3, flags=flags)
    assert np.isfinite(out[0]).all() and np.isnan(out[1]).all()


def test_fp8_cache_doubles_capacity_like_the_pages():
    # Bytes per cached token: BF16 vs e4m3 plus one fp32 scale each for K and V.
    # The pages report ~686k -> ~1.37M tokens for the same memory.
    vals = {}
    with open(os.path.join(GOLDEN, "pages_capacity.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                k, v = line.split()
                vals[k] = float(v)
    lo = vals["fp8_tokens_low"] / vals["bf16_tokens_high"]
    hi = vals["fp8_tokens_high"] / vals["bf16_tokens_low"]
    hkv, d, ps = 8, 128, 64
    pool_bytes = 64 << 30
    per_page_bf16 = 2 * hkv * ps * d * np.dtype(np.uint16).itemsize
    per_page_fp8 = 2 * hkv * ps * d * np.dtype(np.uint8).itemsize
    tokens_bf16 = (pool_bytes // per_page_bf16) * ps
    tokens_fp8 = ((pool_bytes - 8) // per_page_fp8) * ps
    assert lo <= tokens_fp8 / tokens_bf16 <= hi
