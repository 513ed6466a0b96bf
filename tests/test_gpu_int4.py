"""INT4 weight-only decode GEMV on the GPU vs the fp64 oracle, and the
row -> tile weight packing vs the oracle's packing (bit-exact).

Tolerance, per output element (derived from the kernel's arithmetic): the
output is rounded once to BF16, at most 2^-9 |y| away from its fp32 value;
the fp32 evaluation contracts each 128-weight group on the matrix unit with
the codes offset to 1.5 + q/16 (partial sums bounded by 2 sum|x| per group,
a handful of fp32 roundings each), scales the group sum and adds up to
K/128 groups, so its error is a few times 2^-16 sum_k |x_k| s_{g(k)}.  The
bound used is

    |y_gpu - y| <= 2^-8 |y| + 2^-12 sum_k |x_k| s_{g(k)}

which leaves a margin of 2x and ~16x on the two terms.  Sizes span several
groups per wave, ragged N (a padded last tile, an odd number of tiles) and
every count of 16-row activation blocks (M = 1..64), with activations both
staged in LDS (m * k * 2 <= 32 KiB, m <= 16) and read from registers.
"""

import numpy as np
import pytest
import torch

import decode_attention_fp8_kv_amd as fk
from decode_attention_fp8_kv_amd import workloads as W
from oracle import int4_gemv as i4

from parity import say

pytestmark = pytest.mark.gpu


def _np(inp):
    return (W.bits_u16(inp.x), inp.w.cpu().numpy().view(np.uint32), W.bits_u16(inp.scales))


def _check(y_gpu, inp, rows=None):
    x, w, s = _np(inp)
    n = inp.n
    ref = i4.gemv(x, w, s, n)
    srow = i4.scales_from_tiles(s, n, x.shape[1])
    if rows is not None:
        ref, srow, y_gpu = ref[:, rows], srow[rows], y_gpu[:, rows]
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * i4.abs_mass(x, srow)
    err = np.abs(y_gpu - ref)
    worst = float((err / bound).max())
    assert np.all(err <= bound), f"worst error/bound {worst:.3f}"
    return worst


def _run(inp, dev, pad=0):
    m, n = inp.x.shape[0], inp.n
    buf = torch.full((m * n + pad,), -7.0, dtype=torch.bfloat16, device=dev)
    y = buf[:m * n].view(m, n)
    fk.int4_gemv(inp.x.to(dev), inp.w.to(dev), inp.scales.to(dev), y)
    torch.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64), buf[m * n:].cpu()


@pytest.mark.parametrize("m,n,k", [(1, 1, 128), (1, 4096, 4096), (3, 1000, 2048), (16, 257, 1152),
                                   (17, 96, 384), (33, 333, 640), (48, 64, 1024), (64, 500, 2048),
                                   (5, 31, 256), (1, 4100, 16384), (2, 48, 8192), (16, 200, 4096),
                                   # 1,024 tiles: four tiles per workgroup; 1,792: seven
                                   (16, 16384, 1024), (40, 16384, 512), (64, 28672, 256),
                                   # activations in LDS, seven tiles per workgroup (the last one ragged)
                                   (1, 28672, 1024), (3, 28600, 512)])
def test_int4_gemv_matches_oracle(gpu_device, m, n, k):
    say(f"int4_gemv m={m} n={n} k={k}")
    inp = W.make_int4_gemv(m, n, k, seed=m * 1000 + n)
    y, tail = _run(inp, gpu_device, pad=64)
    worst = _check(y, inp)
    assert torch.all(tail.float() == -7.0), "wrote past y"
    say(f"  worst error/bound {worst:.4f}")


@pytest.mark.parametrize("m", [1, 16, 64])
def test_int4_gemv_full_size_sampled_rows(gpu_device, m):
    # the benchmarked projection: 28672 x 8192 (112 MiB of codes); 384 rows checked against the oracle
    n, k = 28672, 8192
    say(f"int4_gemv full size m={m} n={n} k={k}")
    inp = W.make_int4_gemv(m, n, k, seed=77 + m, device=gpu_device)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=gpu_device)
    fk.int4_gemv(inp.x, inp.w, inp.scales, y)
    torch.cuda.synchronize()
    rows = np.sort(np.random.default_rng(m).choice(n, 384, replace=False))
    rows[-1] = n - 1
    cpu = W.Int4GemvInputs(inp.x.cpu(), inp.w.cpu(), inp.scales.cpu(), n)
    _check(y.float().cpu().numpy().astype(np.float64), cpu, rows)


@pytest.mark.parametrize("n,k", [(1, 128), (37, 384), (4096, 2048), (1000, 8192)])
def test_int4_pack_weights_matches_oracle(gpu_device, n, k):
    say(f"int4_pack_weights n={n} k={k}")
    rows = W.make_int4_gemv(1, n, k, seed=n + k, layout="rows")
    ws, ss = fk.int4_tile_shapes(n, k)
    wt = torch.full(ws, 0x5A5A5A5A, dtype=torch.int32, device=gpu_device)
    st = torch.full(ss, 3.0, dtype=torch.bfloat16, device=gpu_device)
    fk.int4_pack_weights(rows.w.to(gpu_device), rows.scales.to(gpu_device), wt, st)
    torch.cuda.synchronize()
    ow, os_ = i4.pack(rows.w.numpy().view(np.uint32), W.bits_u16(rows.scales))
    assert np.array_equal(wt.cpu().numpy().view(np.uint32), ow)
    assert np.array_equal(W.bits_u16(st), os_)


def test_int4_gemv_on_packed_rows_matches_row_oracle(gpu_device):
    say("int4 pack + gemv vs row oracle")
    m, n, k = 4, 300, 1024
    rows = W.make_int4_gemv(m, n, k, seed=5, layout="rows")
    ws, ss = fk.int4_tile_shapes(n, k)
    wt = torch.empty(ws, dtype=torch.int32, device=gpu_device)
    st = torch.empty(ss, dtype=torch.bfloat16, device=gpu_device)
    fk.int4_pack_weights(rows.w.to(gpu_device), rows.scales.to(gpu_device), wt, st)
    y = torch.empty((m, n), dtype=torch.bfloat16, device=gpu_device)
    fk.int4_gemv(rows.x.to(gpu_device), wt, st, y)
    torch.cuda.synchronize()
    x, w, s = W.bits_u16(rows.x), rows.w.numpy().view(np.uint32), W.bits_u16(rows.scales)
    ref = i4.gemv_rows(x, w, s)
    bound = 2.0 ** -8 * np.abs(ref) + 2.0 ** -12 * i4.abs_mass(x, s)
    assert np.all(np.abs(y.float().cpu().numpy() - ref) <= bound)


def test_int4_gemv_extreme_codes_and_scales(gpu_device):
    say("int4_gemv extreme codes")
    m, n, k = 4, 64, 512
    inp = W.make_int4_gemv(m, n, k, seed=3)
    words = inp.w.numpy().view(np.uint32).copy()            # [4 tiles][4 groups][16 rows][16 words]
    words[:, :, 0::4] = 0x88888888          # rows 0, 4, 8, 12 of every tile: all -8
    words[:, :, 1::4] = 0x77777777          # all +7
    words[:, :, 2::4] = 0                   # all 0
    sc = inp.scales.clone()
    sc[0, :, 3] = torch.tensor(2.0 ** 100).to(torch.bfloat16)      # row 3: large but finite products
    sc[0, :, 7] = torch.tensor(2.0 ** -120).to(torch.bfloat16)     # row 7: tiny
    x = inp.x.clone()
    x[1] = x[1].abs()                                              # no cancellation in activation row 1
    e = W.Int4GemvInputs(x, torch.from_numpy(words.view(np.int32)), sc, n)
    y, _ = _run(e, gpu_device)
    _check(y, e)
    assert np.all(y[:, 2::4] == 0.0)


def test_int4_gemv_is_deterministic(gpu_device):
    say("int4_gemv determinism")
    for m in (1, 16):
        inp = W.make_int4_gemv(m, 3000, 4096, seed=9, device=gpu_device)
        ys = []
        for _ in range(3):
            y = torch.empty((m, 3000), dtype=torch.bfloat16, device=gpu_device)
            fk.int4_gemv(inp.x, inp.w, inp.scales, y)
            ys.append(y)
        torch.cuda.synchronize()
        assert torch.equal(ys[0].view(torch.int16), ys[1].view(torch.int16))
        assert torch.equal(ys[0].view(torch.int16), ys[2].view(torch.int16))
