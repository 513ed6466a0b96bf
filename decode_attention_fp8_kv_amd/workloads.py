"""Seeded synthetic workloads for paged decode attention over an FP8 KV cache.

This module only *draws inputs*: lengths, page tables, tags, BF16 K/V/Q rows
and the per-tensor scales that a caller would hand to the append.  It holds
none of the method's arithmetic (no quantization, no attention), imports
neither the HIP binding nor the oracle, and is the one piece of code that
both sides of a parity check share.

The five shapes mirror the workloads of the source pages (Kimi K2.6 decode at
concurrency 1..64, [P1] throughput table / [P3] section "量化 KV 缓存"), at
one GPU's share: 64 query heads over 8 KV heads, head_dim 128, 64-token pages.

Recipes (every random draw comes from a ``torch.Generator`` seeded per field):

* ``tiny``    -- batch 2, 8/2 heads, D 64, pages of 16, lengths 100 and 257,
  K/V/Q ~ N(0,1), a 64-page pool, random uint32 tags with one mismatch
  injected into sequence 1; softmax scale 1/8.
* ``latency`` -- batch 1, context 32768: 32767 tokens cached and the step's
  new token appended at position 32767, so attention covers 32768 tokens in
  a 512-page pool (permuted); all tags valid.
* ``conc32``  -- batch 32, context lengths uniform in [4096, 32768]; 1% of the
  (head, dim) channels of K and of V (10 of 1024) are multiplied by 8; one
  new token per sequence is appended at position ``L0`` and attention runs
  over ``L0 + 1`` tokens; scales come from the cache before the append, so
  appended outliers can saturate.
* ``conc64``  -- batch 64, lengths ``L0`` lognormal (median 12000, sigma 1.0),
  rounded and clipped to [512, 65536]; as in ``conc32`` one new token per
  sequence is appended at ``L0`` and attention covers ``L0 + 1`` tokens; the
  pool holds exactly the pages those lengths need; 0.1% of the pool's pages
  are stale (their tag bumped after the fact).  With
  ``bf16_same_memory=True`` the cache is BF16 in a pool of the same bytes
  (half as many pages): sequences are admitted in order while their pages
  fit -- the first 29 at the default seed -- and 0.1% of that pool's pages
  are stale.
* ``long``    -- batch 8, context 131072 (131071 cached + the step's new
  token), K/V Student-t with 3 degrees of freedom (so e4m3 saturation and
  subnormals occur); the scale is the 99.9th percentile of |x| over a seeded
  2^20-element sample of the cached rows, divided by 448; with
  ``inject_tags=True`` each used (sequence, page) slot independently gets a
  mismatched expected tag with probability 1/1000.

The scale recipe ``amax / 448`` (448 being the largest e4m3 magnitude) is an
input choice made by the caller of the append, not part of the append.

INT4 weight-only GEMV inputs (``make_int4_gemv``): activations x ~ N(0,1)
BF16 [M][K]; weight words uniform random 32-bit patterns (so every 4-bit
code in [-8, 7] is equally likely); scales 2^u BF16 with u uniform in
[-9, -5] (the range of per-group absmax/7 for weights of standard deviation
~0.005..0.05).  No trained weights exist here: the codes are synthetic.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field

import numpy as np
import torch

KV_FP8_E4M3 = 0
KV_BF16 = 1
E4M3_LARGEST = 448.0


@dataclass
class Workload:
    name: str
    batch: int
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    page_size: int
    num_pages: int
    max_pages: int
    seq_lens: np.ndarray            # int32 [B]   tokens attended (context + appended)
    page_table: np.ndarray          # int32 [B][max_pages], -1 where unused
    page_tags: np.ndarray           # uint32 [num_pages]
    expected_tags: np.ndarray       # uint32 [B][max_pages]
    softmax_scale: float            # fp32 value
    k_scale: float                  # fp32 value
    v_scale: float                  # fp32 value
    q: torch.Tensor                 # bf16 [B][Hq][D]
    ctx_k: torch.Tensor             # bf16 [T][Hkv][D]  rows already in the cache
    ctx_v: torch.Tensor
    ctx_seq: torch.Tensor           # int32 [T]
    ctx_pos: torch.Tensor           # int32 [T]
    new_k: torch.Tensor             # bf16 [N][Hkv][D]  rows appended by one decode step
    new_v: torch.Tensor
    new_seq: torch.Tensor           # int32 [N]
    new_pos: torch.Tensor           # int32 [N]
    seed: int = 0
    notes: dict = field(default_factory=dict)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads

    def rows_of(self, b: int):
        """All (context + appended) K and V rows of sequence b, in token order, on CPU."""
        sel = self.ctx_seq == b
        k = self.ctx_k[sel]
        v = self.ctx_v[sel]
        pos = self.ctx_pos[sel]
        nsel = self.new_seq == b
        if bool(nsel.any()):
            k = torch.cat([k, self.new_k[nsel]])
            v = torch.cat([v, self.new_v[nsel]])
            pos = torch.cat([pos, self.new_pos[nsel]])
        order = torch.argsort(pos)
        return k[order].cpu(), v[order].cpu(), pos[order].cpu()


def bits_u16(t: torch.Tensor) -> np.ndarray:
    """A BF16 tensor as a numpy uint16 array of its bit patterns (on CPU)."""
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def _gen(device, seed: int, stream: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed((seed * 1_000_003 + stream * 7919) % (2 ** 63))
    return g


def _cpu_gen(seed: int, stream: int) -> torch.Generator:
    return _gen("cpu", seed, stream)


def _page_layout(lengths, page_size, num_pages, seed):
    """Random physical pages for each sequence, drawn from a permuted pool."""
    g = _cpu_gen(seed, 1)
    n_used = [-(-int(L) // page_size) for L in lengths]
    max_pages = max(n_used)
    perm = torch.randperm(num_pages, generator=g).numpy().astype(np.int32)
    if sum(n_used) > num_pages:
        raise ValueError("pool too small for the requested lengths")
    table = np.full((len(lengths), max_pages), -1, dtype=np.int32)
    i = 0
    for b, n in enumerate(n_used):
        table[b, :n] = perm[i:i + n]
        i += n
    return table, max_pages, n_used


def _tags(table, n_used, num_pages, seed):
    g = _cpu_gen(seed, 2)
    tags = torch.randint(0, 2 ** 32, (num_pages,), generator=g, dtype=torch.int64).numpy().astype(np.uint32)
    expected = np.zeros(table.shape, dtype=np.uint32)
    for b, n in enumerate(n_used):
        expected[b, :n] = tags[table[b, :n]]
    return tags, expected


def _normal(shape, g, device, dtype=torch.float32):
    return torch.randn(shape, generator=g, device=device, dtype=dtype)


def _student_t3(shape, g, device):
    # t_3 = Z / sqrt(chi2_3 / 3), chi2_3 = sum of three squared standard normals
    z = torch.randn(shape, generator=g, device=device)
    c = torch.zeros(shape, device=device)
    for _ in range(3):
        c += torch.randn(shape, generator=g, device=device) ** 2
    return z / torch.sqrt(c / 3.0)


def _rows(lengths, hkv, d, dist, seed, stream, device, outlier_channels=None):
    """BF16 rows for every (sequence, position), concatenated in sequence order."""
    g = _gen(device, seed, stream)
    total = int(sum(lengths))
    out = torch.empty((total, hkv, d), dtype=torch.bfloat16, device=device)
    chunk = 1 << 16
    for s in range(0, total, chunk):
        n = min(chunk, total - s)
        x = _student_t3((n, hkv, d), g, device) if dist == "t3" else _normal((n, hkv, d), g, device)
        if outlier_channels is not None:
            x.view(n, hkv * d)[:, outlier_channels] *= 8.0
        out[s:s + n] = x.to(torch.bfloat16)
    seq = torch.repeat_interleave(torch.arange(len(lengths), dtype=torch.int32),
                                  torch.as_tensor(lengths, dtype=torch.int64)).to(device)
    pos = torch.cat([torch.arange(int(L), dtype=torch.int32) for L in lengths]).to(device)
    return out, seq, pos


def _amax_scale(*tensors) -> float:
    amax = max(float(t.abs().amax()) for t in tensors if t.numel())
    return float(np.float32(amax / E4M3_LARGEST))


def _quantile_scale(t: torch.Tensor, q: float, seed: int) -> float:
    g = _gen(t.device.type, seed, 9)
    flat = t.view(-1)
    idx = torch.randint(0, flat.numel(), (1 << 20,), generator=g, device=t.device)
    sample = flat[idx].float().abs()
    return float(np.float32(float(torch.quantile(sample, q)) / E4M3_LARGEST))


CONFIG_NAMES = ("tiny", "latency", "conc32", "conc64", "long")
DEFAULT_SEEDS = {"tiny": 1, "latency": 2, "conc32": 3, "conc64": 4, "long": 5}


def make(name: str, seed: int | None = None, device="cpu", *, bf16_same_memory=False,
         inject_tags=False, batch=None, context=None, long_scale="p999") -> Workload:
    """Build workload ``name`` on ``device`` ("cpu" or "cuda").

    ``batch`` / ``context`` shrink a configuration for quick tests (same
    recipe, fewer or shorter sequences); the full sizes are the defaults.
    ``long_scale="amax"`` gives ``long`` the amax / 448 scale instead of the
    99.9th percentile (nothing saturates; many small values become
    subnormal codes).
    """
    seed = DEFAULT_SEEDS[name] if seed is None else seed
    dev = torch.device(device)
    notes = {}
    new_rows = False
    outliers = None
    dist = "normal"

    if name == "tiny":
        B, hq, hkv, d, ps = 2, 8, 2, 64, 16
        ctx = np.array([100, 257], dtype=np.int64)
        num_pages = 64
        sm = 1.0 / math.sqrt(64)
    else:
        hq, hkv, d, ps = 64, 8, 128, 64
        sm = 1.0 / math.sqrt(128)
        g = _cpu_gen(seed, 0)
        if name == "latency":
            B = 1 if batch is None else batch
            ctx = np.full(B, (32768 if context is None else context) - 1, dtype=np.int64)
            new_rows = True
        elif name == "conc32":
            B = 32 if batch is None else batch
            hi = 32768 if context is None else context
            lo = min(4096, hi)
            ctx = torch.randint(lo, hi + 1, (B,), generator=g).numpy().astype(np.int64)
            new_rows = True
            gch = _cpu_gen(seed, 3)
            n_out = round(0.01 * hkv * d)
            outliers = (torch.randperm(hkv * d, generator=gch)[:n_out],
                        torch.randperm(hkv * d, generator=gch)[:n_out])
            notes["outlier_channels"] = n_out
        elif name == "conc64":
            B = 64 if batch is None else batch
            z = torch.randn(B, generator=g, dtype=torch.float64).numpy()
            ctx = np.rint(np.exp(math.log(12000.0) + 1.0 * z)).astype(np.int64)
            ctx = np.clip(ctx, 512, 65536 if context is None else context)
            new_rows = True
        elif name == "long":
            B = 8 if batch is None else batch
            ctx = np.full(B, (131072 if context is None else context) - 1, dtype=np.int64)
            dist = "t3"
            new_rows = True
        else:
            raise KeyError(name)
        n_att = ctx + (1 if new_rows else 0)
        need = int(sum(-(-int(L) // ps) for L in n_att))
        num_pages = need          # the pool holds exactly the pages in use
        if name == "conc64" and bf16_same_memory:
            # a BF16 page holds twice the bytes of an FP8 one: the same memory holds half the pages;
            # sequences are admitted in order while their pages fit
            num_pages = need // 2
            pages = np.array([-(-int(L) // ps) for L in n_att])
            admitted = int(np.searchsorted(np.cumsum(pages), num_pages, side="right"))
            ctx = ctx[:admitted]
            B = admitted
            notes["admitted"] = admitted

    att_lens = ctx + (1 if new_rows else 0)
    table, max_pages, n_used = _page_layout(att_lens, ps, num_pages, seed)
    tags, expected = _tags(table, n_used, num_pages, seed)

    if name == "tiny":
        gi = _cpu_gen(seed, 4)
        b_bad = 1
        j = int(torch.randint(0, n_used[b_bad], (1,), generator=gi))
        expected[b_bad, j] ^= 1
        notes["mismatch"] = (b_bad, j)
    if name == "conc64":
        gi = _cpu_gen(seed, 4)
        n_stale = max(1, round(0.001 * num_pages))
        stale = torch.randperm(num_pages, generator=gi)[:n_stale].numpy()
        tags[stale] += np.uint32(1)
        notes["stale_pages"] = int(n_stale)
    if name == "long" and inject_tags:
        gi = _cpu_gen(seed, 4)
        hit = torch.rand(table.shape, generator=gi).numpy() < 1e-3
        used = np.arange(max_pages)[None, :] < np.array(n_used)[:, None]
        hit &= used
        expected[hit] ^= np.uint32(1)
        notes["injected"] = int(hit.sum())

    k_out = v_out = None
    if outliers is not None:
        k_out, v_out = outliers
        k_out, v_out = k_out.to(dev), v_out.to(dev)
    ctx_k, ctx_seq, ctx_pos = _rows(ctx, hkv, d, dist, seed, 10, dev, k_out)
    ctx_v, _, _ = _rows(ctx, hkv, d, dist, seed, 11, dev, v_out)

    if name == "long" and long_scale == "p999":
        k_scale = _quantile_scale(ctx_k, 0.999, seed)
        v_scale = _quantile_scale(ctx_v, 0.999, seed + 1)
    else:
        k_scale = _amax_scale(ctx_k)
        v_scale = _amax_scale(ctx_v)

    if new_rows:
        nk, nseq, _ = _rows(np.ones(B, np.int64), hkv, d, dist, seed, 12, dev, k_out)
        nv, _, _ = _rows(np.ones(B, np.int64), hkv, d, dist, seed, 13, dev, v_out)
        npos = torch.as_tensor(ctx, dtype=torch.int32).to(dev)
    else:
        nk = torch.empty((0, hkv, d), dtype=torch.bfloat16, device=dev)
        nv = nk.clone()
        nseq = torch.empty(0, dtype=torch.int32, device=dev)
        npos = nseq.clone()

    gq = _gen(dev.type, seed, 14)
    q = _normal((B, hq, d), gq, dev).to(torch.bfloat16)

    return Workload(
        name=name, batch=B, num_q_heads=hq, num_kv_heads=hkv, head_dim=d, page_size=ps,
        num_pages=num_pages, max_pages=max_pages,
        seq_lens=att_lens.astype(np.int32), page_table=table, page_tags=tags,
        expected_tags=expected, softmax_scale=float(np.float32(sm)),
        k_scale=k_scale, v_scale=v_scale, q=q,
        ctx_k=ctx_k, ctx_v=ctx_v, ctx_seq=ctx_seq, ctx_pos=ctx_pos,
        new_k=nk, new_v=nv, new_seq=nseq, new_pos=npos, seed=seed, notes=notes)


def kv_bytes(w: Workload, kv_dtype: int, flags=None) -> int:
    """Algorithmic bytes one decode call must move for the non-aborted sequences.

    K and V rows (``2 * L * Hkv * D * e``), the query and the output
    (``2 * Hq * D * 2``), the page-table entry plus page tag plus expected tag
    for each used page (12 bytes), and the abort-flag byte.
    """
    e = 1 if kv_dtype == KV_FP8_E4M3 else 2
    total = 0
    for b in range(w.batch):
        if flags is not None and flags[b]:
            continue
        L = int(w.seq_lens[b])
        total += 2 * L * w.num_kv_heads * w.head_dim * e
        total += 2 * w.num_q_heads * w.head_dim * 2
        total += (-(-L // w.page_size)) * 12
    return total + w.batch


def make_custom(lengths, num_q_heads, num_kv_heads, head_dim, page_size, *, num_pages=None, seed=0,
                dist="normal", device="cpu", mismatch=(), spare_pages=3, softmax_scale=None,
                q_scale=1.0) -> Workload:
    """A small workload of any supported shape, for parity tests.

    ``lengths`` are the tokens attended per sequence (all already cached);
    the pool gets ``spare_pages`` unused pages beyond those needed (or exactly
    ``num_pages``); ``mismatch`` lists (sequence, page slot) pairs whose
    expected tag is flipped; ``dist`` is "normal" or "t3".
    """
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    need = int(sum(-(-int(L) // page_size) for L in lengths))
    num_pages = need + spare_pages if num_pages is None else num_pages
    dev = torch.device(device)
    table, max_pages, n_used = _page_layout(np.maximum(lengths, 1), page_size, num_pages, seed)
    tags, expected = _tags(table, n_used, num_pages, seed)
    for b, j in mismatch:
        expected[b, j] ^= np.uint32(1)
    ctx_k, ctx_seq, ctx_pos = _rows(lengths, num_kv_heads, head_dim, dist, seed, 10, dev)
    ctx_v, _, _ = _rows(lengths, num_kv_heads, head_dim, dist, seed, 11, dev)
    k_scale, v_scale = _amax_scale(ctx_k), _amax_scale(ctx_v)
    gq = _gen(dev.type, seed, 14)
    q = (_normal((B, num_q_heads, head_dim), gq, dev) * q_scale).to(torch.bfloat16)
    sm = 1.0 / math.sqrt(head_dim) if softmax_scale is None else softmax_scale
    empty = torch.empty((0, num_kv_heads, head_dim), dtype=torch.bfloat16, device=dev)
    none = torch.empty(0, dtype=torch.int32, device=dev)
    return Workload(
        name="custom", batch=B, num_q_heads=num_q_heads, num_kv_heads=num_kv_heads, head_dim=head_dim,
        page_size=page_size, num_pages=num_pages, max_pages=max_pages,
        seq_lens=lengths.astype(np.int32), page_table=table, page_tags=tags, expected_tags=expected,
        softmax_scale=float(np.float32(sm)), k_scale=k_scale, v_scale=v_scale, q=q,
        ctx_k=ctx_k, ctx_v=ctx_v, ctx_seq=ctx_seq, ctx_pos=ctx_pos,
        new_k=empty, new_v=empty.clone(), new_seq=none, new_pos=none.clone(), seed=seed)


@dataclass
class Int4GemvInputs:
    x: torch.Tensor        # bf16 [M][K]
    w: torch.Tensor        # int32 codes: tile layout [ceil(N/16)][K/128][16][16], or row layout [N][K/8]
    scales: torch.Tensor   # bf16: tile layout [ceil(N/16)][K/128][16], or row layout [N][K/128]
    n: int


def make_int4_gemv(m: int, n: int, k: int, seed: int = 0, device="cpu", layout: str = "tiles") -> Int4GemvInputs:
    """Seeded INT4 GEMV inputs (recipe in the module docstring).  Random
    words are valid codes in either layout; in the tile layout the padding
    rows hold random codes too (a GEMV must not let them reach an output)."""
    if k % 128 != 0:
        raise ValueError("k must be a multiple of 128")
    t, g = -(-n // 16), k // 128
    wshape, sshape = ((t, g, 16, 16), (t, g, 16)) if layout == "tiles" else ((n, k // 8), (n, g))
    x = torch.randn((m, k), generator=_gen(device, seed, 101), device=device).to(torch.bfloat16)
    w = torch.randint(-2 ** 31, 2 ** 31, wshape, generator=_gen(device, seed, 102), device=device,
                      dtype=torch.int64).to(torch.int32)
    u = torch.rand(sshape, generator=_gen(device, seed, 103), device=device) * 4.0 - 9.0
    scales = torch.exp2(u).to(torch.bfloat16)
    return Int4GemvInputs(x.contiguous(), w.contiguous(), scales.contiguous(), n)
