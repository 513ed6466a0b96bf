#!/usr/bin/env python3
"""Benchmark: decode-attention tokens/s and effective KV GB/s on one MI355X.

One step = the whole decode hot path for one batch: ``kv_quant_append`` of
the step's new K/V rows (one token per sequence) followed by
``paged_decode_attn`` over the paged FP8 e4m3 cache with the page-tag check
on.  The workload is the batch-32 concurrency case (64 query / 8 KV heads,
head_dim 128, 64-token pages, context lengths uniform in [4096, 32768], 1% of
channels scaled x8), synthetic and seeded, resident in HBM before timing.

Printed: one JSON line.  ``value`` = FP8 decode tokens/s (sequences decoded
per second, one token each, for one attention layer); the BF16-cache run of
the same workload is reported beside it, plus the tag-check overhead, the
roofline of the decode kernel (algorithmic bytes per launch / mean launch
time from HIP events on the launch stream) and the CPU oracle's rate on a
bounded sample of the same workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --workload latency|conc64|long --decode-only   (the other
      configurations: the same decode legs, FP8 and BF16, without the
      page-pool, hand-off, INT4 and CPU legs)
  python bench.py --summarize-profiles OUT   (writes profiles/ from rocprofv3 runs)
"""

from __future__ import annotations

import argparse
import hashlib
import json
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_HBM_GBPS = 8000.0          # MI355X HBM3E peak, GB/s
WORKLOAD = "conc32"             # the default workload (the headline line)
WORKLOADS = {
    "conc32": ("conc32: batch 32, 64 q heads / 8 KV heads, head_dim 128, page 64, context U[4096,32768] "
               "+ 1 appended token per step, page-tag check on",
               "synthetic (seeded; K/V/Q ~ N(0,1) bf16, 1% channels x8, random page permutation)"),
    "latency": ("latency: batch 1, 64 q heads / 8 KV heads, head_dim 128, page 64, context 32768, "
                "page-tag check on",
                "synthetic (seeded; K/V/Q ~ N(0,1) bf16, random page permutation)"),
    "conc64": ("conc64: batch 64, 64 q heads / 8 KV heads, head_dim 128, page 64, context lognormal "
               "(median 12000, sigma 1) clipped to [512, 65536], pool exactly full, 0.1% of pages stale "
               "(their sequences abort and are not counted); the BF16 run uses the first 32 sequences",
               "synthetic (seeded; K/V/Q ~ N(0,1) bf16, random page permutation, stale page tags)"),
    "long": ("long: batch 8, 64 q heads / 8 KV heads, head_dim 128, page 64, context 131072, "
             "page-tag check on",
             "synthetic (seeded; K/V Student-t nu=3 bf16, scale p99.9/448, Q ~ N(0,1), random page permutation)"),
}
PROFILE_COUNTERS = os.path.join(ROOT, "profiles", "decode_kernel_conc32_fp8_counters.txt")
KERNEL_SOURCES = ["decode_attention_fp8_kv_amd/csrc/decode_attn.hip", "decode_attention_fp8_kv_amd/csrc/common.hpp",
                  "decode_attention_fp8_kv_amd/csrc/internal.hpp", "decode_attention_fp8_kv_amd/csrc/api.cpp"]


INT4_SOURCES = ["decode_attention_fp8_kv_amd/csrc/int4_gemv.hip", "decode_attention_fp8_kv_amd/csrc/common.hpp"]


def kernel_source_hash(sources=None) -> str:
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def algorithmic_bytes(w, kv_dtype, flags=None) -> int:
    """Bytes one decode call must move at minimum for the non-aborted sequences:
    K and V rows (2*L*Hkv*D*e), q and out (2*Hq*D*2), the page-table entry,
    page tag and expected tag of every used page (12 B each), one flag byte."""
    e = 1 if kv_dtype == 0 else 2
    total = 0
    for b in range(w.batch):
        if flags is not None and flags[b]:
            continue
        L = int(w.seq_lens[b])
        total += 2 * L * w.num_kv_heads * w.head_dim * e + 2 * w.num_q_heads * w.head_dim * 2
        total += (-(-L // w.page_size)) * 12
    return total + w.batch


class Case:
    """A workload resident on the GPU with its cache filled in one KV dtype."""

    def __init__(self, w, kv_dtype, dev):
        import torch
        import decode_attention_fp8_kv_amd as fk

        self.fk, self.torch, self.w, self.kv, self.dev = fk, torch, w, kv_dtype, dev
        shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
        dt = torch.uint8 if kv_dtype == fk.KV_FP8_E4M3 else torch.bfloat16
        self.kc = torch.zeros(shape, dtype=dt, device=dev)
        self.vc = torch.zeros(shape, dtype=dt, device=dev)
        self.pt = torch.from_numpy(w.page_table).to(dev)
        self.lens = torch.from_numpy(w.seq_lens).to(dev)
        self.tags = torch.from_numpy(w.page_tags.view(np.int32)).to(dev)
        self.exp = torch.from_numpy(w.expected_tags.view(np.int32)).to(dev)
        self.q = w.q.to(dev).contiguous()
        self.out = torch.empty_like(self.q)
        self.flags = torch.empty(w.batch, dtype=torch.uint8, device=dev)
        self.ws = fk.alloc_workspace(w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim, w.page_size,
                                     w.max_pages, device=dev)
        # Bulk fill of the cache (every context row), timed on its second run
        # (the first one also loads the kernel's code object).
        fill_ms = []
        for _ in range(2):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fk.kv_quant_append(w.ctx_k, w.ctx_v, w.ctx_seq, w.ctx_pos, self.pt, w.k_scale, w.v_scale,
                               self.kc, self.vc, kv_dtype)
            b.record()
            torch.cuda.synchronize(dev)
            fill_ms.append(a.elapsed_time(b))
        n_el = 2 * w.ctx_k.numel()                   # K and V elements
        per_el = 3 if kv_dtype == fk.KV_FP8_E4M3 else 4  # bf16 read + cache element written
        self.fill = {"rows": int(w.ctx_k.shape[0]), "us": round(fill_ms[-1] * 1e3, 1),
                     "gbps": round(n_el * per_el / (fill_ms[-1] * 1e-3) / 1e9, 1),
                     "bytes_per_element": per_el}
        self.new = (w.new_k.contiguous(), w.new_v.contiguous(), w.new_seq, w.new_pos)
        torch.cuda.synchronize(dev)

    def append(self):
        nk, nv, ns, npos = self.new
        self.fk.kv_quant_append(nk, nv, ns, npos, self.pt, self.w.k_scale, self.w.v_scale, self.kc, self.vc,
                                self.kv)

    def decode(self, tags=True):
        w = self.w
        self.fk.paged_decode_attn(self.q, self.kc, self.vc, self.pt, self.lens, self.out, self.flags, self.ws,
                                  kv_dtype=self.kv, k_scale=w.k_scale, v_scale=w.v_scale,
                                  page_tags=self.tags if tags else None,
                                  expected_tags=self.exp if tags else None, softmax_scale=w.softmax_scale)

    def step(self):
        self.append()
        self.decode(tags=True)


def time_steps(case, steps, warmup, every=4):
    """Warm up, then time exactly `steps` steps between two synchronizations
    with nothing else on the stream: the wall clock over them gives the
    throughput.  A second pass of `steps` steps, outside that timed region,
    brackets every `every`-th step with three HIP events on the launch
    stream -- before its append, after its append, after its decode -- which
    give the per-call durations.  Events stay out of the timed steps because
    each recorded event costs the step a few microseconds of wall time
    (measured 225 / 231 / 238 us per step with 0 / 2 / 3 events on every
    step at Conc-32) while leaving the bracketed durations unchanged.  The
    default warm-up (300 steps) outlasts the GPU's climb back to full speed
    after the host-side setup: after one second idle, Conc-32 steps took
    322 us for the first 20, 222.5 us over the next 200 and 220.8 us from
    then on (measured)."""
    torch = case.torch
    for _ in range(warmup):
        case.step()
    torch.cuda.synchronize(case.dev)
    t0 = time.perf_counter()
    for _ in range(steps):
        case.step()
    torch.cuda.synchronize(case.dev)
    wall = time.perf_counter() - t0
    n_samples = (steps + every - 1) // every
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(n_samples)]
    for i in range(steps):
        if i % every == 0:
            e0, e1, e2 = evs[i // every]
            e0.record()
            case.append()
            e1.record()
            case.decode(tags=True)
            e2.record()
        else:
            case.append()
            case.decode(tags=True)
    torch.cuda.synchronize(case.dev)
    app_ms = np.array([e0.elapsed_time(e1) for e0, e1, _ in evs])
    dec_ms = np.array([e1.elapsed_time(e2) for _, e1, e2 in evs])
    return wall, dec_ms, app_ms


def time_flushed(case, iters=30, flush_bytes=1 << 30):
    """Per-call protocol: before each timed call, outside the timed region, a
    1 GiB read evicts the 256 MB Infinity Cache and the L2s (a read, not a
    write: a 1 GiB write would leave up to 256 MB of dirty lines that the
    timed call then pays to write back); HIP events bracket the single call.
    Returns (median, p95) in microseconds."""
    torch = case.torch
    scratch = torch.ones(flush_bytes, dtype=torch.uint8, device=case.dev)
    sink = torch.empty(1, dtype=torch.uint8, device=case.dev)
    for _ in range(5):
        case.decode(True)
    ms = []
    for _ in range(iters):
        sink[0] = scratch.max()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        case.decode(True)
        b.record()
        torch.cuda.synchronize(case.dev)
        ms.append(a.elapsed_time(b))
    del scratch, sink
    return round(float(np.median(ms)) * 1e3, 2), round(float(np.percentile(ms, 95)) * 1e3, 2)


def tag_overhead(case, iters=100):
    """Decode-only launch times with tags on vs off, interleaved."""
    torch = case.torch
    on, off = [], []
    for _ in range(5):
        case.decode(True)
        case.decode(False)
    for i in range(iters):
        for tags, dst in ((True, on), (False, off)) if i % 2 == 0 else ((False, off), (True, on)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            case.decode(tags)
            b.record()
            dst.append((a, b))
    torch.cuda.synchronize(case.dev)
    on_ms = np.array([a.elapsed_time(b) for a, b in on])
    off_ms = np.array([a.elapsed_time(b) for a, b in off])
    return {
        "median_on_us": round(float(np.median(on_ms)) * 1e3, 2),
        "median_off_us": round(float(np.median(off_ms)) * 1e3, 2),
        "p95_on_us": round(float(np.percentile(on_ms, 95)) * 1e3, 2),
        "p95_off_us": round(float(np.percentile(off_ms, 95)) * 1e3, 2),
        "overhead_median": round(float(np.median(on_ms) / np.median(off_ms) - 1.0), 4),
        "overhead_p95": round(float(np.percentile(on_ms, 95) / np.percentile(off_ms, 95) - 1.0), 4),
    }


def copy_bandwidth(dev, nbytes=2 << 30, reps=10):
    """Device-to-device copy of `nbytes` (read + write counted): the box's
    practical streaming rate, reported beside the roofline, never in its place.
    Its kernel is also the plain copy of known size used to scale the
    FETCH_SIZE / WRITE_SIZE counters."""
    import torch

    src = torch.empty(nbytes, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize(dev)
    gbps = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return gbps


def pool_timings(dev, batch=32, max_pages=513, reps=20):
    """Median HIP-event time of the page-pool calls at the benchmark's shape:
    a decode step's growth (one page for each of 32 sequences), a prefill's
    (512 pages each), freeing all 32 sequences, and a 32-row checked append.
    All are single small kernels, so they are reported in microseconds."""
    import torch
    import decode_attention_fp8_kv_amd as fk

    num_pages = batch * max_pages
    free_pages = torch.empty(num_pages, dtype=torch.int32, device=dev)
    free_count = torch.empty(1, dtype=torch.int32, device=dev)
    counts = torch.zeros(batch, dtype=torch.int32, device=dev)
    table = torch.full((batch, max_pages), -1, dtype=torch.int32, device=dev)
    expected = torch.zeros((batch, max_pages), dtype=torch.int32, device=dev)
    tags = torch.zeros(num_pages, dtype=torch.int32, device=dev)
    status = torch.empty(batch, dtype=torch.uint8, device=dev)
    one = torch.ones(batch, dtype=torch.int32, device=dev)
    prefill = torch.full((batch,), 512, dtype=torch.int32, device=dev)
    release = torch.ones(batch, dtype=torch.uint8, device=dev)

    def timed(fn):
        ms = []
        for _ in range(reps):
            fk.page_pool_init(free_pages, free_count)
            counts.zero_()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn()
            b.record()
            torch.cuda.synchronize(dev)
            ms.append(a.elapsed_time(b))
        return round(float(np.median(ms)) * 1e3, 2)

    res = {
        "alloc_32x1_us": timed(lambda: fk.page_alloc(one, counts, table, expected, tags, free_pages, free_count,
                                                       status)),
        "alloc_32x512_us": timed(lambda: fk.page_alloc(prefill, counts, table, expected, tags, free_pages,
                                                         free_count, status)),
    }

    def alloc_then_free():
        fk.page_alloc(prefill, counts, table, expected, tags, free_pages, free_count, status)
        torch.cuda.synchronize(dev)
    ms = []
    for _ in range(reps):
        fk.page_pool_init(free_pages, free_count)
        counts.zero_()
        alloc_then_free()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        fk.page_free(release, counts, table, free_pages, free_count, status)
        b.record()
        torch.cuda.synchronize(dev)
        ms.append(a.elapsed_time(b))
    res["free_32x512_us"] = round(float(np.median(ms)) * 1e3, 2)
    return res


def handoff_timings(dev, reps=10):
    """Prefill -> decode hand-off of a 32,768-token prefill (64/8 heads, head_dim
    128, 64-token pages): device amax + scale of K and of V (one
    kv_absmax_scale_kv call; two kv_absmax_scale calls beside it), then the
    device-scale append into the FP8 pool.  Median of `reps` after a warm-up;
    GB/s at 2 bytes per element read (amax) and 3 per element (append)."""
    import torch
    import decode_attention_fp8_kv_amd as fk
    from decode_attention_fp8_kv_amd import workloads as W

    w = W.make("latency", device=dev)
    k, v = w.ctx_k.contiguous(), w.ctx_v.contiguous()
    shape = (w.num_pages, w.num_kv_heads, w.page_size, w.head_dim)
    kc = torch.empty(shape, dtype=torch.uint8, device=dev)
    vc = torch.empty(shape, dtype=torch.uint8, device=dev)
    pt = torch.from_numpy(w.page_table).to(dev)
    kvs = torch.zeros(4, device=dev)
    work = torch.empty(2 * fk.AMAX_WORK_FLOATS, device=dev)
    ev = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(reps + 2)]
    for e in ev:
        e[0].record()
        fk.kv_absmax_scale_kv(k, v, kvs, work)      # both scales, one reduction + one finish launch
        e[1].record()
        fk.kv_quant_append_dscale(k, v, w.ctx_seq, w.ctx_pos, pt, kvs[1:2], kvs[3:4], kc, vc)
        e[2].record()
    # the same amax with one call per tensor, for comparison
    ks, vs = torch.zeros(2, device=dev), torch.zeros(2, device=dev)
    ev1 = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps + 2)]
    for e in ev1:
        e[0].record()
        fk.kv_absmax_scale(k, ks, work)
        fk.kv_absmax_scale(v, vs, work)
        e[1].record()
    torch.cuda.synchronize(dev)
    amax_ms = float(np.median([a.elapsed_time(b) for a, b, _ in ev[2:]]))
    app_ms = float(np.median([b.elapsed_time(c) for _, b, c in ev[2:]]))
    single_ms = float(np.median([a.elapsed_time(b) for a, b in ev1[2:]]))
    n = k.numel() + v.numel()
    return {"tokens": int(k.shape[0]), "amax_scale_us": round(amax_ms * 1e3, 1),
            "amax_gbps": round(2 * n / (amax_ms * 1e-3) / 1e9, 1),
            "amax_scale_two_calls_us": round(single_ms * 1e3, 1), "append_us": round(app_ms * 1e3, 1),
            "append_gbps": round(3 * n / (app_ms * 1e-3) / 1e9, 1),
            "total_us": round((amax_ms + app_ms) * 1e3, 1)}


def int4_gemv_timings(dev, n=28672, k=8192, nbuf=8, reps=10, ms=(1, 16, 64)):
    """INT4 weight-only decode GEMV y = x W^T over an n x k projection
    (28672 x 8192: 112 MiB of 4-bit codes + 3.5 MiB of scales), M activation
    rows.  Calls rotate over `nbuf` distinct weight sets (896 MiB, larger than
    the Infinity Cache), so every call streams its weights from HBM.  Mean
    over `reps` rounds after a warm-up; GB/s at the algorithmic bytes (codes
    n*k/2 + scales n*k/64 + x 2*m*k + y 2*m*n).  The BF16 GEMV of the same
    shape (torch.matmul, 4x the weight bytes) is timed the same way for
    context."""
    import torch
    import decode_attention_fp8_kv_amd as fk
    from decode_attention_fp8_kv_amd import workloads as W

    bufs = [W.make_int4_gemv(max(ms), n, k, seed=s, device=dev) for s in range(nbuf)]
    out = {"shape": f"{n} x {k}", "weight_sets": nbuf, "group": 128}
    for m in ms:
        xs = [b.x[:m].contiguous() for b in bufs]
        ys = [torch.empty((m, n), dtype=torch.bfloat16, device=dev) for _ in range(nbuf)]
        for i in range(2 * nbuf):
            fk.int4_gemv(xs[i % nbuf], bufs[i % nbuf].w, bufs[i % nbuf].scales, ys[i % nbuf])
        torch.cuda.synchronize(dev)
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        for _ in range(reps):
            for i in range(nbuf):
                fk.int4_gemv(xs[i], bufs[i].w, bufs[i].scales, ys[i])
        b.record()
        torch.cuda.synchronize(dev)
        us = a.elapsed_time(b) * 1e3 / (reps * nbuf)
        alg = n * k // 2 + n * (k // 128) * 2 + 2 * m * k + 2 * m * n
        out[f"m{m}"] = {"us": round(us, 2), "gbps": round(alg / (us * 1e-6) / 1e9, 1),
                        "pct_hbm_peak": round(100.0 * alg / (us * 1e-6) / 1e9 / PEAK_HBM_GBPS, 2)}
    del bufs
    wb = [torch.randn((n, k), device=dev, dtype=torch.bfloat16) for _ in range(2)]
    x1 = torch.randn((1, k), device=dev, dtype=torch.bfloat16)
    for _ in range(3):
        for wt in wb:
            torch.matmul(x1, wt.t())
    torch.cuda.synchronize(dev)
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        for wt in wb:
            torch.matmul(x1, wt.t())
    b.record()
    torch.cuda.synchronize(dev)
    us = a.elapsed_time(b) * 1e3 / (2 * reps)
    out["bf16_weights_torch_m1"] = {"us": round(us, 2), "gbps": round(2 * n * k / (us * 1e-6) / 1e9, 1)}
    out["int4_over_bf16_speed_m1"] = round(us / out["m1"]["us"], 2)
    del wb
    torch.cuda.empty_cache()
    return out


def cpu_baseline(w, budget_s=15.0):
    """The CPU oracle, as it stands, on a bounded sample of the same workload:
    for whole sequences taken in order, time one decode step (append of the new
    row, tag check, fp64 attention over the page-table-gathered FP8 cache)."""
    from threadpoolctl import threadpool_info

    from decode_attention_fp8_kv_amd import workloads as W
    from oracle import paged_attn as pa

    done, elapsed, tokens = [], 0.0, 0
    for b in range(w.batch):
        L = int(w.seq_lens[b])
        n = -(-L // w.page_size)
        k, v, pos = w.rows_of(b)
        shape = (n, w.num_kv_heads, w.page_size, w.head_dim)
        kc, vc = np.zeros(shape, np.uint8), np.zeros(shape, np.uint8)
        mini_pt = np.arange(n, dtype=np.int32)[None, :]
        ctx = pos.numpy() < L - 1                                   # the cache before this step
        pa.append(W.bits_u16(k[ctx]), W.bits_u16(v[ctx]), np.zeros(int(ctx.sum()), np.int32), pos.numpy()[ctx],
                  mini_pt, w.k_scale, w.v_scale, kc, vc)
        tags = w.page_tags[w.page_table[b, :n]]
        exp = w.expected_tags[b:b + 1, :n]
        q = W.bits_u16(w.q[b:b + 1])
        t0 = time.perf_counter()
        pa.append(W.bits_u16(k[~ctx]), W.bits_u16(v[~ctx]), np.zeros(int((~ctx).sum()), np.int32),
                  pos.numpy()[~ctx], mini_pt, w.k_scale, w.v_scale, kc, vc)
        flags = pa.abort_flags(mini_pt, np.array([L]), w.page_size, n, tags, exp)
        pa.decode_attention(q, kc, vc, pa.KV_FP8_E4M3, w.k_scale, w.v_scale, mini_pt, np.array([L]),
                            w.softmax_scale, flags=flags)
        elapsed += time.perf_counter() - t0
        done.append(b)
        tokens += L
        if elapsed >= budget_s:
            break
    threads = max([p.get("num_threads", 1) for p in threadpool_info()] + [1])
    cpu_model = "unknown"
    try:
        with open("/proc/cpuinfo") as f:
            for ln in f:
                if ln.startswith("model name"):
                    cpu_model = ln.split(":", 1)[1].strip()
                    break
    except OSError:
        pass
    return {
        "value": round(len(done) / elapsed, 3),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "sample": f"{len(done)} of {w.batch} sequences ({tokens} cached tokens), one decode step each, "
                  f"{elapsed:.1f} s of CPU time; numpy fp64 with {threads} BLAS threads",
    }


PROFILE_TRACE = os.path.join(ROOT, "profiles", "decode_kernel_conc32_fp8_trace.md")
PROFILE_INT4 = os.path.join(ROOT, "profiles", "int4_gemv_28672x8192_counters.md")
INT4_INSTANCES = {1: "int4_gemv_kernel<1, 7, 2, true>", 16: "int4_gemv_kernel<1, 7, 2, false>",
                  64: "int4_gemv_kernel<4, 7, 2, false>"}
PROFILE_CMDS = {
    "trace": "rocprofv3 --kernel-trace --stats -f csv -d OUT/trace -o run -- "
             "python3 bench.py --steps 20 --warmup 5 --no-cpu-baseline",
    "trace_wl": "rocprofv3 --kernel-trace --stats -f csv -d OUT/trace_{wl} -o run -- "
                "python3 bench.py --workload {wl} --decode-only --steps 40 --warmup 5",
    "fetch": "rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/pmc_fetch -o run -- "
             "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-bf16",
    "write": "rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/pmc_write -o run -- "
             "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-bf16",
    "sq": "rocprofv3 --pmc SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_LDS_BANK_CONFLICT SQ_INSTS_VMEM_RD "
          "SQ_WAVES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY -f csv -d OUT/pmc_sq -o run -- "
          "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-bf16",
    "tcc": "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum -f csv -d OUT/pmc_tcc -o run -- "
           "python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-bf16",
    "lds": "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS SQ_LDS_ADDR_CONFLICT SQ_LDS_IDX_ACTIVE -f csv "
           "-d OUT/pmc_lds -o run -- python3 bench.py --steps 5 --warmup 2 --no-cpu-baseline --no-bf16",
}
PROFILE_SQ = os.path.join(ROOT, "profiles", "decode_kernel_conc32_fp8_sq_tcc_counters.txt")
COPY_BYTES = 2 << 30            # the device copy of copy_bandwidth(): the counters' calibration


def summarize_profiles(out_dir: str) -> None:
    """Write the committed text summaries from the three rocprofv3 runs in
    PROFILE_CMDS (run from the repository root, OUT = out_dir).  The counter
    pass reads FETCH_SIZE / WRITE_SIZE in KiB per dispatch; each is scaled by
    bytes / counter of the 2 GiB device copy measured in the same run."""
    import csv
    from collections import defaultdict

    def rows(path):
        with open(path) as f:
            return list(csv.DictReader(f))

    stats = rows(os.path.join(out_dir, "trace", "run_kernel_stats.csv"))
    keep = [r for r in stats if "fp8kv" in r["Name"]]
    lines = ["# Kernel trace of bench.py: paged_decode_attn on the conc32 workload (FP8 and BF16 KV), plus the "
             "append, page pool, hand-off and INT4 GEMV legs", "",
             "Command (from the repository root; OUT is any output folder):", "",
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["trace"], "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    avg = {}
    def short(kname):
        kname = kname.replace("void ", "").replace("fp8kv::(anonymous namespace)::", "")
        return re.sub(r"\(.*\)$", "", kname)

    for r in keep:
        name = short(r["Name"])
        avg[name] = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{name}` | {r['Calls']} | {avg[name]:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    dec = avg.get("decode_kernel<0, 128, 16, true>")
    mrg = next((v for k, v in avg.items() if k.startswith("merge_kernel<128")), None)
    chk = next((v for k, v in avg.items() if k.startswith("check_kernel")), None)
    if dec is not None and mrg is not None and chk is not None:
        lines += ["", f"One FP8 `paged_decode_attn` call = check_kernel + decode_kernel<0, 128, 16, true> + "
                      f"merge_kernel<128, 1> = {chk:.2f} + {dec:.2f} + {mrg:.2f} = {chk + dec + mrg:.2f} us of kernel "
                      f"time (the check and merge averages cover the FP8 and BF16 calls).",
                  "decode_kernel<0,...> is the FP8-cache instance, decode_kernel<1,...> the BF16 one; "
                  "quant_append_kernel<0>/<1> are kv_quant_append (their averages mix the 32-row appends of the "
                  "timed steps with the two bulk fills of the whole cache before timing)."]
    lines.append("")
    with open(PROFILE_TRACE, "w") as f:
        f.write("\n".join(lines))

    per = {}
    for key, counter in (("fetch", "FETCH_SIZE"), ("write", "WRITE_SIZE")):
        vals = defaultdict(list)
        for r in rows(os.path.join(out_dir, f"pmc_{key}", "run_counter_collection.csv")):
            if r["Counter_Name"] == counter:
                vals[r["Kernel_Name"]].append(float(r["Counter_Value"]))
        copy = [v for k, v in vals.items() if "copyBuffer" in k for v in v]
        big = [v for v in copy if v >= 0.9 * max(copy)]
        factor = COPY_BYTES / (sum(big) / len(big) * 1024.0)
        dk = [v for k, v in vals.items() if "decode_kernel<0, 128, 16, true>" in k for v in v]
        mk = [v for k, v in vals.items() if "merge_kernel<128" in k for v in v]
        ck = [v for k, v in vals.items() if "check_kernel" in k for v in v]
        per[key] = (factor, sum(dk) / len(dk), sum(mk) / len(mk), sum(ck) / len(ck), len(dk), len(big))
    ff, fd, fm, fc, nd, nc = per["fetch"]
    wf, wd, wm, wc, _, _ = per["write"]
    traffic = (fd + fm + fc) * 1024.0 * ff + (wd + wm + wc) * 1024.0 * wf
    from decode_attention_fp8_kv_amd import workloads as W
    w = W.make(WORKLOAD)
    alg = algorithmic_bytes(w, 0)
    out = [
        "# HBM traffic of one FP8 paged_decode_attn call (check_kernel + decode_kernel<0, 128, 16, true> +",
        "# merge_kernel<128, 1>)",
        "# on the conc32 workload, from two rocprofv3 counter passes (from the repository root; OUT is any folder):",
        "#   export TMPDIR=/tmp && " + PROFILE_CMDS["fetch"],
        "#   export TMPDIR=/tmp && " + PROFILE_CMDS["write"],
        "# Counters are KiB per dispatch; each is scaled by bytes / counter of the 2 GiB device copy",
        "# (__amd_rocclr_copyBuffer) that bench.py runs in the same process.",
        f"kernel_source_hash: {kernel_source_hash()}",
        f"decode_dispatches: {nd}",
        f"copy_dispatches: {nc}",
        f"fetch_kib_per_dispatch_decode: {fd:.1f}",
        f"fetch_kib_per_dispatch_merge: {fm:.1f}",
        f"fetch_kib_per_dispatch_check: {fc:.1f}",
        f"write_kib_per_dispatch_decode: {wd:.1f}",
        f"write_kib_per_dispatch_merge: {wm:.1f}",
        f"write_kib_per_dispatch_check: {wc:.1f}",
        f"fetch_scale: {ff:.4f}",
        f"write_scale: {wf:.4f}",
        f"traffic_bytes_per_launch: {traffic:.0f}",
        f"algorithmic_bytes_per_launch: {alg}",
        f"traffic_over_algorithmic: {traffic / alg:.4f}",
        "",
    ]
    with open(PROFILE_COUNTERS, "w") as f:
        f.write("\n".join(out))

    # INT4 GEMV: the instances bench.py's int4_gemv_timings runs (M = 1, 16, 64 on 28672 x 8192)
    n_, k_ = 28672, 8192
    fetch = defaultdict(list)
    write = defaultdict(list)
    for key, counter, dst in (("fetch", "FETCH_SIZE", fetch), ("write", "WRITE_SIZE", write)):
        for r in rows(os.path.join(out_dir, f"pmc_{key}", "run_counter_collection.csv")):
            if r["Counter_Name"] == counter and "int4_gemv_kernel" in r["Kernel_Name"]:
                dst[short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    lines = ["# INT4 weight-only GEMV on a 28672 x 8192 projection (bench.py's int4_gemv leg)", "",
             "Commands (from the repository root; OUT is any output folder):", "",
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["trace"],
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["fetch"],
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["write"], "",
             "Average kernel time from the trace; FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by the "
             "2 GiB device copy's factors above; algorithmic bytes = codes n*k/2 + scales n*k/64 + "
             "x 2*m*k + y 2*m*n.", "",
             "| M | kernel | average us | algorithmic MB | HBM MB (fetch + write) | traffic / algorithmic | "
             "GB/s (algorithmic / average) |",
             "|---|---|---|---|---|---|---|"]
    for m_, kname in INT4_INSTANCES.items():
        if kname not in avg or not fetch.get(kname) or not write.get(kname):
            continue
        alg4 = n_ * k_ // 2 + n_ * (k_ // 128) * 2 + 2 * m_ * k_ + 2 * m_ * n_
        hbm = (sum(fetch[kname]) / len(fetch[kname]) * ff + sum(write[kname]) / len(write[kname]) * wf) * 1024.0
        lines.append(f"| {m_} | `{kname}` | {avg[kname]:.2f} | {alg4 / 1e6:.1f} | {hbm / 1e6:.1f} | "
                     f"{hbm / alg4:.3f} | {alg4 / (avg[kname] * 1e-6) / 1e9:.0f} |")
    lines += ["", f"kernel_source_hash: {kernel_source_hash(INT4_SOURCES)} (int4_gemv.hip, common.hpp)", ""]
    with open(PROFILE_INT4, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {PROFILE_TRACE}, {PROFILE_COUNTERS} and {PROFILE_INT4}")
    if os.path.isdir(os.path.join(out_dir, "pmc_sq")) and os.path.isdir(os.path.join(out_dir, "pmc_tcc")):
        summarize_sq_tcc(out_dir, short)
    for wl in ("latency", "conc64", "long"):
        if os.path.isdir(os.path.join(out_dir, f"trace_{wl}")):
            summarize_workload_trace(out_dir, wl, short)


def summarize_workload_trace(out_dir: str, wl: str, short) -> None:
    """Kernel times of one paged_decode_attn call (check + decode + merge) on
    another workload, from a rocprofv3 kernel trace of bench.py --workload."""
    import csv
    with open(os.path.join(out_dir, f"trace_{wl}", "run_kernel_stats.csv")) as f:
        stats = [r for r in csv.DictReader(f) if "fp8kv" in r["Name"]]
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{wl}_trace.md")
    lines = [f"# Kernel trace of bench.py on the {wl} workload (FP8 and BF16 KV, decode legs only)", "",
             WORKLOADS[wl][0] + ".", "",
             "Command (from the repository root; OUT is any output folder):", "",
             f"    export TMPDIR=/tmp && {PROFILE_CMDS['trace_wl'].format(wl=wl)}", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    avg = {}
    for r in stats:
        name = short(r["Name"])
        avg[name] = float(r["AverageNs"]) / 1e3
        lines.append(f"| `{name}` | {r['Calls']} | {avg[name]:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    chk = next((v for k, v in avg.items() if k.startswith("check_kernel")), None)
    mrg = [k for k in avg if k.startswith("merge_kernel")]
    for kv, dec in (("FP8", "decode_kernel<0, 128, 16, true>"), ("BF16", "decode_kernel<1, 128, 16, true>")):
        if dec in avg and chk is not None and mrg:
            m = avg[mrg[0]]
            lines.append("")
            lines.append(f"One {kv} call = check_kernel + `{dec}` + `{mrg[0]}` = {chk:.2f} + {avg[dec]:.2f} + "
                         f"{m:.2f} = {chk + avg[dec] + m:.2f} us of kernel time (check and merge averaged over "
                         f"both dtypes).")
    lines += ["", f"kernel_source_hash: {kernel_source_hash()}", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {path}")


def summarize_sq_tcc(out_dir: str, short) -> None:
    """Instruction mix, LDS conflicts and L2 hit rate of the FP8 decode kernel (per dispatch)."""
    import csv
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(float))
    for sub_dir in ("pmc_sq", "pmc_tcc", "pmc_lds"):
        if not os.path.isdir(os.path.join(out_dir, sub_dir)):
            continue
        with open(os.path.join(out_dir, sub_dir, "run_counter_collection.csv")) as f:
            for r in csv.DictReader(f):
                if short(r["Kernel_Name"]) == "decode_kernel<0, 128, 16, true>":
                    vals[r["Counter_Name"]][(sub_dir, r["Dispatch_Id"])] += float(r["Counter_Value"])
    avg = {k: sum(d.values()) / len(d) for k, d in vals.items() if d}
    from decode_attention_fp8_kv_amd import workloads as W
    w = W.make(WORKLOAD)
    tiles = sum(-(-int(L) // 64) for L in w.seq_lens) * w.num_kv_heads   # (sequence, KV head, 64-token tile)
    out = ["# decode_kernel<0, 128, 16, true> (FP8 cache) on the conc32 workload: instruction mix, LDS bank",
           "# conflicts and L2 hits, per dispatch, from two rocprofv3 counter passes (repository root; OUT any folder):",
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["sq"],
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["tcc"],
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["lds"],
           "# (a counter read in two passes is averaged over both)",
           f"kernel_source_hash: {kernel_source_hash()}",
           f"tiles_per_dispatch: {tiles}   # (sequence, KV head, 64-token tile) triples"]
    for k in sorted(avg):
        out.append(f"{k}: {avg[k]:.0f}")
    if "SQ_INSTS_MFMA" in avg:
        out.append(f"mfma_per_tile: {avg['SQ_INSTS_MFMA'] / tiles:.2f}")
    if "SQ_INSTS_VALU" in avg:
        out.append(f"valu_per_tile: {avg['SQ_INSTS_VALU'] / tiles:.1f}")
    if avg.get("SQ_INSTS_LDS"):
        out.append(f"lds_bank_conflict_cycles_per_lds_instruction: "
                   f"{avg.get('SQ_LDS_BANK_CONFLICT', 0.0) / avg['SQ_INSTS_LDS']:.3f}")
        out.append(f"lds_bank_conflict_cycles_per_tile: {avg.get('SQ_LDS_BANK_CONFLICT', 0.0) / tiles:.1f}   "
                   f"# against a tile period of ~2,500 cycles per wave: not a limit")
    if avg.get("TCC_HIT_sum", 0) + avg.get("TCC_MISS_sum", 0) > 0:
        out.append(f"l2_hit_rate: {avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.4f}")
    out.append("")
    with open(PROFILE_SQ, "w") as f:
        f.write("\n".join(out))
    print(f"wrote {PROFILE_SQ}")


def main():
    if len(sys.argv) == 3 and sys.argv[1] == "--summarize-profiles":
        summarize_profiles(sys.argv[2])
        return
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawDescriptionHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=300)
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-bf16", action="store_true")
    ap.add_argument("--no-copy", action="store_true", help="skip the device-copy bandwidth measurement")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=WORKLOAD,
                    help="decode workload (default: the batch-32 headline)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the decode legs: no copy, page-pool, hand-off, INT4 or CPU measurements")
    args = ap.parse_args()
    if args.decode_only:
        args.no_copy = args.no_cpu_baseline = True
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: decode sequences shard across GPUs with no exchange "
              "between them, and no multi-GPU run is made.", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_fp8_kv_amd as fk
    from decode_attention_fp8_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    fk.load_library()
    copy_gbps = None if args.no_copy else copy_bandwidth(dev)
    w = W.make(args.workload, device=dev)
    res = {}
    for kv, name in ((fk.KV_FP8_E4M3, "fp8"), (fk.KV_BF16, "bf16")):
        if name == "bf16" and args.no_bf16:
            continue
        # the BF16 run of the full-pool workload takes the first 32 sequences (a BF16 cache of all 64 would
        # not fit the pool the FP8 cache fills)
        wk = W.make(args.workload, device=dev, bf16_subset=True) if (name == "bf16" and
                                                                     args.workload == "conc64") else w
        case = Case(wk, kv, dev)
        torch.cuda.synchronize(dev)
        wall, dec_ms, app_ms = time_steps(case, args.steps, args.warmup)
        flags = case.flags.cpu().numpy()
        alg = algorithmic_bytes(wk, kv, flags)
        ok = int((flags == 0).sum())
        mean_us = float(dec_ms.mean()) * 1e3
        res[name] = {
            "value": ok * args.steps / wall,
            "ms_per_step": wall / args.steps * 1e3,
            "decode_mean_us": mean_us,
            "decode_median_us": float(np.median(dec_ms)) * 1e3,
            "decode_p95_us": float(np.percentile(dec_ms, 95)) * 1e3,
            "alg_bytes": alg,
            "gbps": alg / (mean_us * 1e-6) / 1e9,
            "aborted": int(wk.batch - ok),
            "append_median_us": float(np.median(app_ms)) * 1e3,
            "fill": case.fill,
            "flushed": time_flushed(case),
        }
        if name == "fp8" and "stale_pages" not in wk.notes:
            res["tags"] = tag_overhead(case)
        elif name == "fp8":
            # with stale tags, turning the check off changes the work (nothing aborts): no like-for-like
            res["tags"] = {"skipped": "the workload has stale page tags; tags off would decode the aborted sequences"}
        if name == "fp8" and w.new_k.shape[0] > 0:
            # the step's append, with the tag check of the page's owner
            rs = torch.empty(w.new_k.shape[0], dtype=torch.uint8, device=dev)
            nk, nv, ns, npos = case.new
            evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(20)]
            for a, b in evs:   # back to back like the step loop's appends
                a.record()
                fk.kv_quant_append_checked(nk, nv, ns, npos, case.pt, w.k_scale, w.v_scale, case.kc, case.vc,
                                           case.tags, case.exp, rs)
                b.record()
            torch.cuda.synchronize(dev)
            res["append_checked_us"] = float(np.median([a.elapsed_time(b) for a, b in evs])) * 1e3
        del case
        torch.cuda.empty_cache()

    f = res["fp8"]
    traffic = None
    if os.path.exists(PROFILE_COUNTERS):
        prof = {}
        with open(PROFILE_COUNTERS) as fh:
            for ln in fh:
                if ":" in ln and not ln.startswith("#"):
                    key, val = ln.split(":", 1)
                    prof[key.strip()] = val.strip()
        if (args.workload == WORKLOAD and prof.get("kernel_source_hash") == kernel_source_hash()
                and "traffic_bytes_per_launch" in prof):
            traffic = int(float(prof["traffic_bytes_per_launch"]))
    line = {
        "metric": "decode-attn tokens/s + effective KV GB/s (% HBM peak), FP8 vs BF16 KV, 1 GPU",
        "value": round(f["value"], 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(f["ms_per_step"], 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3",
        "data": WORKLOADS[args.workload][1],
        "config": {
            "workload": WORKLOADS[args.workload][0],
            "batch": w.batch, "num_q_heads": w.num_q_heads, "num_kv_heads": w.num_kv_heads,
            "head_dim": w.head_dim, "page_size": w.page_size, "context_tokens": int(w.seq_lens.sum()),
            "parallelism": "single GPU",
        },
        "effective_kv_gbps": round(f["gbps"], 1),
        "pct_hbm_peak": round(100.0 * f["gbps"] / PEAK_HBM_GBPS, 2),
        "decode_us": {"mean": round(f["decode_mean_us"], 2), "median": round(f["decode_median_us"], 2),
                      "p95": round(f["decode_p95_us"], 2)},
        "roofline": {
            "kernel": "paged_decode_attn FP8: check_kernel + decode_kernel<0,128,16,true> + merge_kernel<128,1>",
            "bound": "hbm",
            "achieved": round(f["gbps"], 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(f["gbps"] / PEAK_HBM_GBPS, 4),
            "traffic": traffic,
        },
        "tag_check": res.get("tags"),
        "decode_us_flushed": {"median": f["flushed"][0], "p95": f["flushed"][1],
                              "protocol": "1 GiB read before each call (evicts the Infinity Cache), "
                                          "outside the timed region; 30 calls"},
        "bulk_fill": f["fill"],
        "device_copy_gbps": None if copy_gbps is None else round(copy_gbps, 1),
    }
    if w.new_k.shape[0] > 0:
        line["append_32_rows_us"] = round(f["append_median_us"], 2)
        line["append_checked_32_rows_us"] = round(res["append_checked_us"], 2)
    if not args.decode_only:
        line["page_pool"] = pool_timings(dev)
        line["prefill_handoff"] = handoff_timings(dev)
        line["int4_gemv"] = int4_gemv_timings(dev)
    if "bf16" in res:
        b = res["bf16"]
        line["bf16"] = {"value": round(b["value"], 1), "unit": "tokens/s", "ms_per_step": round(b["ms_per_step"], 4),
                        "effective_kv_gbps": round(b["gbps"], 1),
                        "pct_hbm_peak": round(100.0 * b["gbps"] / PEAK_HBM_GBPS, 2),
                        "decode_mean_us": round(b["decode_mean_us"], 2)}
        line["fp8_over_bf16_tokens_per_s"] = round(f["value"] / b["value"], 3)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(w)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
