#!/usr/bin/env python3
"""Benchmark: decode-attention tokens/s and effective KV GB/s on one MI355X.

One step = the whole decode hot path for one batch, as one
``paged_decode_step`` call: the step's new K/V rows (one token per sequence)
quantized and appended to the paged FP8 e4m3 cache, with the page-tag check
in the same launch, then the split decode over the cache and the merge.  The
headline workload is the concurrency-64 case at a full pool (64 query / 8 KV
heads, head_dim 128, 64-token pages, context lengths lognormal with median
12,000 clipped to [512, 65536], the pool exactly the pages those lengths
need, 0.1% of its pages stale so the sequences using them abort), synthetic
and seeded, resident in HBM before timing.

Printed: one JSON line.  ``value`` = FP8 decode tokens/s (sequences decoded
per second, one token each, for one attention layer; aborted sequences do not
count).  Beside it: the BF16-cache run in a pool of the same bytes (it admits
29 of the 64 sequences), the roofline of the decode kernel (algorithmic bytes
per launch / mean kernel time from HIP events recorded right before and after
it on the launch stream), the whole step's time, the other workloads (batch
32, batch 1 at 32k, batch 8 at 131k) with the same figures, the tag-check
overhead against calls with no check at all, the legs of the page pool, the
prefill hand-off and the INT4 GEMV, and the CPU oracle's rate on a bounded
sample of the headline workload.

  python bench.py [--gpus 1] [--steps K] [--warmup W] [--no-cpu-baseline]
  python bench.py --workload conc64|conc32|latency|long --decode-only
      (one workload's FP8 and BF16 legs only: what the profiles trace)
  python bench.py --next-only   (the page-pool, hand-off and INT4 legs only)
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
WORKLOAD = "conc64"             # the headline workload
EXTRA_WORKLOADS = ("conc32", "long", "latency")
TAG_AB_WORKLOADS = ("conc32", "long")   # tags on vs off; conc64 has stale pages (off would change the work)
WORKLOADS = {
    "conc64": ("conc64: batch 64, 64 q heads / 8 KV heads, head_dim 128, page 64, context L0 lognormal "
               "(median 12000, sigma 1) clipped to [512, 65536] + 1 appended token per step, pool exactly the "
               "pages needed, 0.1% of pages stale (their sequences abort and are not counted), page-tag check on; "
               "BF16 leg: a pool of the same bytes, sequences admitted in order while they fit",
               "synthetic (seeded; K/V/Q ~ N(0,1) bf16, random page permutation, stale page tags)"),
    "conc32": ("conc32: batch 32, 64 q heads / 8 KV heads, head_dim 128, page 64, context U[4096,32768] "
               "+ 1 appended token per step, page-tag check on",
               "synthetic (seeded; K/V/Q ~ N(0,1) bf16, 1% channels x8, random page permutation)"),
    "latency": ("latency: batch 1, 64 q heads / 8 KV heads, head_dim 128, page 64, context 32768 (the last "
                "token appended by the step), page-tag check on",
                "synthetic (seeded; K/V/Q ~ N(0,1) bf16, random page permutation)"),
    "long": ("long: batch 8, 64 q heads / 8 KV heads, head_dim 128, page 64, context 131072 (the last token "
             "appended by the step), page-tag check on",
             "synthetic (seeded; K/V Student-t nu=3 bf16, scale p99.9/448, Q ~ N(0,1), random page permutation)"),
}
DECODE_KERNEL = {0: "decode_kernel<0, 128, 16, true>", 1: "decode_kernel<1, 128, 16, true>"}
KERNEL_SOURCES = ["decode_attention_fp8_kv_amd/csrc/decode_attn.hip", "decode_attention_fp8_kv_amd/csrc/common.hpp",
                  "decode_attention_fp8_kv_amd/csrc/internal.hpp", "decode_attention_fp8_kv_amd/csrc/api.cpp",
                  "decode_attention_fp8_kv_amd/csrc/page_check.hpp",
                  "decode_attention_fp8_kv_amd/csrc/quant_append.hip"]
INT4_SOURCES = ["decode_attention_fp8_kv_amd/csrc/int4_gemv.hip", "decode_attention_fp8_kv_amd/csrc/common.hpp"]


def counters_path(wl: str, kv_name: str) -> str:
    return os.path.join(ROOT, "profiles", f"decode_kernel_{wl}_{kv_name}_counters.txt")


def _code_only(text: str) -> str:
    """C/C++/HIP source without its comments and with whitespace runs collapsed:
    what the compiler sees, so that a comment edit does not invalidate a profile."""
    out, i, n = [], 0, len(text)
    while i < n:
        c = text[i]
        if c in "\"'":                            # string or character literal, kept whole
            j = i + 1
            while j < n and text[j] != c:
                j += 2 if text[j] == "\\" else 1
            out.append(text[i:j + 1])
            i = j + 1
        elif text.startswith("//", i):
            j = text.find("\n", i)
            i = n if j < 0 else j
        elif text.startswith("/*", i):
            j = text.find("*/", i + 2)
            out.append(" ")
            i = n if j < 0 else j + 2
        else:
            out.append(c)
            i += 1
    return " ".join("".join(out).split())


def kernel_source_hash(sources=None) -> str:
    """Hash of the kernel sources' code (comments and layout ignored)."""
    h = hashlib.sha256()
    for rel in sources or KERNEL_SOURCES:
        with open(os.path.join(ROOT, rel), encoding="utf-8") as f:
            h.update(_code_only(f.read()).encode())
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


def append_bytes(w, kv_dtype) -> int:
    """Bytes of the step's append: each new K/V element read as BF16 and written as one cache
    element, plus the row's sequence index and position."""
    n = int(w.new_k.numel())
    e = 1 if kv_dtype == 0 else 2
    return 2 * n * (2 + e) + 8 * int(w.new_k.shape[0])


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
        # Bulk fill of the cache (every context row), timed in steady state
        # like the decode: the median of runs 10-12 (the first one also loads
        # the kernel's code object, and the first few fills of a process run
        # up to ~10% slower than later ones).
        fill_ms = []
        for _ in range(12):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fk.kv_quant_append(w.ctx_k, w.ctx_v, w.ctx_seq, w.ctx_pos, self.pt, w.k_scale, w.v_scale,
                               self.kc, self.vc, kv_dtype)
            b.record()
            torch.cuda.synchronize(dev)
            fill_ms.append(a.elapsed_time(b))
        n_el = 2 * w.ctx_k.numel()                   # K and V elements
        per_el = 3 if kv_dtype == fk.KV_FP8_E4M3 else 4  # bf16 read + cache element written
        fill = sorted(fill_ms[9:])[1]
        self.fill = {"rows": int(w.ctx_k.shape[0]), "us": round(fill * 1e3, 1),
                     "gbps": round(n_el * per_el / (fill * 1e-3) / 1e9, 1),
                     "bytes_per_element": per_el, "timing": "median of runs 10-12 of the same fill"}
        self.new = (w.new_k.contiguous(), w.new_v.contiguous(), w.new_seq, w.new_pos)
        torch.cuda.synchronize(dev)

    def step(self, tags=True, events=None):
        """One paged_decode_step: append the step's rows, page check (tags on), decode, merge."""
        w = self.w
        nk, nv, ns, npos = self.new
        self.fk.paged_decode_step(nk, nv, ns, npos, self.q, self.kc, self.vc, self.pt, self.lens, self.out,
                                  self.flags, self.ws, kv_dtype=self.kv, k_scale=w.k_scale, v_scale=w.v_scale,
                                  page_tags=self.tags if tags else None, expected_tags=self.exp if tags else None,
                                  softmax_scale=w.softmax_scale, decode_events=events)

    def decode(self, tags=True):
        """paged_decode_attn alone (with tags on: check kernel, decode, merge; off: decode, merge)."""
        w = self.w
        self.fk.paged_decode_attn(self.q, self.kc, self.vc, self.pt, self.lens, self.out, self.flags, self.ws,
                                  kv_dtype=self.kv, k_scale=w.k_scale, v_scale=w.v_scale,
                                  page_tags=self.tags if tags else None,
                                  expected_tags=self.exp if tags else None, softmax_scale=w.softmax_scale)


def time_steps(case, steps, warmup, every=4):
    """Warm up, then time exactly `steps` steps between two synchronizations
    with nothing else on the stream: the wall clock over them gives the
    throughput.  A second pass of `steps` steps, outside that timed region,
    brackets every `every`-th step with four HIP events on the launch stream:
    before the step, right before its decode kernel, right after it (both
    recorded by the library inside the step) and after the step -- the step's
    and the decode kernel's durations.  Events stay out of the timed steps
    because each recorded event costs the step a few microseconds of wall
    time.  The default warm-up (300 steps) outlasts the GPU's climb back to
    full speed after the host-side setup: after one second idle, batch-32
    steps took 322 us for the first 20, 222.5 us over the next 200 and
    220.8 us from then on (measured)."""
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
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_samples)]
    for e in evs:   # create the events outside the sampled steps
        for x in e:
            x.record()
    torch.cuda.synchronize(case.dev)
    for i in range(steps):
        if i % every == 0:
            e0, e1, e2, e3 = evs[i // every]
            e0.record()
            case.step(events=(e1, e2))
            e3.record()
        else:
            case.step()
    torch.cuda.synchronize(case.dev)
    step_ms = np.array([e0.elapsed_time(e3) for e0, _, _, e3 in evs])
    dec_ms = np.array([e1.elapsed_time(e2) for _, e1, e2, _ in evs])
    return wall, step_ms, dec_ms


def time_flushed(case, iters=30, flush_bytes=1 << 30):
    """Per-step protocol: before each timed step, outside the timed region, a
    1 GiB read evicts the 256 MB Infinity Cache and the L2s (a read, not a
    write: a 1 GiB write would leave up to 256 MB of dirty lines that the
    timed step then pays to write back); HIP events bracket the single step.
    Returns (median, p95) in microseconds."""
    torch = case.torch
    scratch = torch.ones(flush_bytes, dtype=torch.uint8, device=case.dev)
    sink = torch.empty(1, dtype=torch.uint8, device=case.dev)
    for _ in range(5):
        case.step()
    ms = []
    for _ in range(iters):
        sink[0] = scratch.max()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record()
        case.step()
        b.record()
        torch.cuda.synchronize(case.dev)
        ms.append(a.elapsed_time(b))
    del scratch, sink
    return round(float(np.median(ms)) * 1e3, 2), round(float(np.percentile(ms, 95)) * 1e3, 2)


def _ab(case, fn, iters):
    """fn(True) vs fn(False), interleaved (the order alternates), HIP events around each."""
    torch = case.torch
    on, off = [], []
    for _ in range(10):
        fn(True)
        fn(False)
    for i in range(iters):
        for tags, dst in ((True, on), (False, off)) if i % 2 == 0 else ((False, off), (True, on)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record()
            fn(tags)
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


def tag_overhead(case, iters=200):
    """The tag check's cost against calls that run no check at all (tags off:
    no page-check work, the decode range-checks the page ids it loads anyway).
    ``step``: paged_decode_step with tags on (page check in the append's
    launch) vs off.  ``call``: paged_decode_attn with tags on (a page-check
    kernel of its own before the decode) vs off."""
    return {"step": _ab(case, lambda t: case.step(tags=t), iters),
            "call": _ab(case, case.decode, iters),
            "protocol": f"{iters} tags-on and {iters} tags-off runs interleaved, HIP events around each; "
                        "tags off = no page check of any kind beyond the decode's own page-id range check"}


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


def read_traffic(wl, kv_name):
    """HBM bytes per decode-kernel launch from the committed counter summary, if it
    was taken on the current kernel sources; else None."""
    path = counters_path(wl, kv_name)
    if not os.path.exists(path):
        return None
    prof = {}
    with open(path) as fh:
        for ln in fh:
            if ":" in ln and not ln.startswith("#"):
                key, val = ln.split(":", 1)
                prof[key.strip()] = val.split("#")[0].strip()
    if prof.get("kernel_source_hash") != kernel_source_hash() or "decode_traffic_bytes_per_launch" not in prof:
        return None
    return int(float(prof["decode_traffic_bytes_per_launch"]))


def run_workload(wl, dev, steps, warmup, *, bf16=True, flushed=False, tag_ab=False):
    """Both KV dtypes of one workload: step throughput, step and decode-kernel times,
    rooflines; optionally the evicted-cache protocol and the tag A/B (FP8)."""
    import torch
    import decode_attention_fp8_kv_amd as fk
    from decode_attention_fp8_kv_amd import workloads as W

    res = {}
    for kv, name in ((fk.KV_FP8_E4M3, "fp8"), (fk.KV_BF16, "bf16")):
        if name == "bf16" and not bf16:
            continue
        wk = W.make(wl, device=dev, bf16_same_memory=(name == "bf16" and wl == "conc64"))
        case = Case(wk, kv, dev)
        torch.cuda.synchronize(dev)
        wall, step_ms, dec_ms = time_steps(case, steps, warmup)
        flags = case.flags.cpu().numpy()
        alg = algorithmic_bytes(wk, kv, flags)
        alg_step = alg + append_bytes(wk, kv)
        ok = int((flags == 0).sum())
        dec_us, step_us = float(dec_ms.mean()) * 1e3, float(step_ms.mean()) * 1e3
        r = {
            "value": ok * steps / wall,
            "ms_per_step": wall / steps * 1e3,
            "batch": wk.batch, "aborted": int(wk.batch - ok), "context_tokens": int(wk.seq_lens.sum()),
            "num_pages": wk.num_pages,
            "decode_kernel_us": {"mean": dec_us, "median": float(np.median(dec_ms)) * 1e3,
                                 "p95": float(np.percentile(dec_ms, 95)) * 1e3},
            "step_us": {"mean": step_us, "median": float(np.median(step_ms)) * 1e3,
                        "p95": float(np.percentile(step_ms, 95)) * 1e3},
            "alg_bytes": alg, "alg_bytes_step": alg_step,
            "decode_gbps": alg / (dec_us * 1e-6) / 1e9,
            "step_gbps": alg_step / (step_us * 1e-6) / 1e9,
            "wall_gbps": alg_step * steps / wall / 1e9,
            "fill": case.fill,
            "traffic": read_traffic(wl, name),
        }
        if flushed and name == "fp8":
            r["flushed"] = time_flushed(case)
        if tag_ab and name == "fp8":
            r["tag_check"] = tag_overhead(case)
        res[name] = r
        del case
        torch.cuda.empty_cache()
    return res


def _round(x, n=2):
    return None if x is None else round(float(x), n)


def summary(r):
    """The per-dtype keys reported for a workload."""
    out = {"tokens_per_s": _round(r["value"], 1), "ms_per_step": _round(r["ms_per_step"], 4),
           "batch": r["batch"], "aborted": r["aborted"], "context_tokens": r["context_tokens"],
           "decode_kernel_us": {k: _round(v) for k, v in r["decode_kernel_us"].items()},
           "step_us": {k: _round(v) for k, v in r["step_us"].items()},
           "alg_bytes_decode": r["alg_bytes"], "alg_bytes_step": r["alg_bytes_step"],
           "decode_kernel_gbps": _round(r["decode_gbps"], 1),
           "decode_kernel_frac": _round(r["decode_gbps"] / PEAK_HBM_GBPS, 4),
           "step_gbps": _round(r["step_gbps"], 1), "step_frac": _round(r["step_gbps"] / PEAK_HBM_GBPS, 4),
           "wall_frac": _round(r["wall_gbps"] / PEAK_HBM_GBPS, 4),
           "decode_traffic_bytes": r["traffic"],
           "bulk_fill": r["fill"]}
    if "tag_check" in r:
        out["tag_check"] = r["tag_check"]
    return out


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
    if "m1" in out:
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

    done, elapsed, tokens, decoded = [], 0.0, 0, 0
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
        decoded += int(flags[0] == 0)
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
        "value": round(decoded / elapsed, 3),
        "unit": "tokens/s",
        "cores": int(threads),
        "kind": "oracle",
        "cpu_model": cpu_model,
        "affinity_cores": len(os.sched_getaffinity(0)),
        "sample": f"{len(done)} of {w.batch} sequences in order ({tokens} tokens, {len(done) - decoded} aborted by "
                  f"the tag check and not counted), one decode step each (append of the new row, tag check, fp64 "
                  f"attention), {elapsed:.1f} s of CPU time; numpy fp64 with {threads} BLAS threads",
    }


PROFILE_INT4 = os.path.join(ROOT, "profiles", "int4_gemv_28672x8192_counters.md")
PROFILE_NEXT = os.path.join(ROOT, "profiles", "next_rows_trace.md")
INT4_INSTANCES = {1: "int4_gemv_kernel<1, 7, 2, true>", 16: "int4_gemv_kernel<1, 7, 2, false>",
                  64: "int4_gemv_kernel<4, 7, 2, false>"}
PROFILE_CMDS = {
    "trace_wl": "rocprofv3 --kernel-trace --stats -f csv -d OUT/trace_{wl} -o run -- "
                "python3 bench.py --workload {wl} --decode-only --no-tag-ab",
    "fetch_wl": "rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/pmc_fetch_{wl} -o run -- "
                "python3 bench.py --workload {wl} --decode-only --no-tag-ab --steps 10 --warmup 5 "
                "--json-out OUT/pmc_fetch_{wl}/line.json",
    "write_wl": "rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/pmc_write_{wl} -o run -- "
                "python3 bench.py --workload {wl} --decode-only --no-tag-ab --steps 10 --warmup 5",
    "trace_next": "rocprofv3 --kernel-trace --stats -f csv -d OUT/trace_next -o run -- python3 bench.py --next-only",
    "fetch_next": "rocprofv3 --pmc FETCH_SIZE -f csv -d OUT/pmc_fetch_next -o run -- python3 bench.py --next-only",
    "write_next": "rocprofv3 --pmc WRITE_SIZE -f csv -d OUT/pmc_write_next -o run -- python3 bench.py --next-only",
    "sq": "rocprofv3 --pmc SQ_INSTS_MFMA SQ_INSTS_VALU SQ_INSTS_LDS SQ_INSTS_VMEM_RD "
          "SQ_WAVES SQ_WAIT_INST_ANY SQ_ACTIVE_INST_ANY -f csv -d OUT/pmc_sq -o run -- "
          "python3 bench.py --workload conc64 --decode-only --no-tag-ab --no-bf16 --steps 10 --warmup 5",
    "lds": "rocprofv3 --pmc SQ_LDS_BANK_CONFLICT SQ_INSTS_LDS -f csv -d OUT/pmc_lds -o run -- "
           "python3 bench.py --workload conc64 --decode-only --no-tag-ab --no-bf16 --steps 10 --warmup 5",
    "tcc": "rocprofv3 --pmc TCC_HIT_sum TCC_MISS_sum TCC_EA0_RDREQ_sum -f csv -d OUT/pmc_tcc -o run -- "
           "python3 bench.py --workload conc64 --decode-only --no-tag-ab --no-bf16 --steps 10 --warmup 5",
}
PROFILE_SQ = os.path.join(ROOT, "profiles", "decode_kernel_conc64_fp8_sq_tcc_counters.txt")
COPY_BYTES = 2 << 30            # the device copy of copy_bandwidth(): the counters' calibration


def _short(kname: str) -> str:
    kname = kname.replace("void ", "").replace("fp8kv::(anonymous namespace)::", "")
    return re.sub(r"\(.*\)$", "", kname)


def _csv_rows(path):
    import csv
    with open(path) as f:
        return list(csv.DictReader(f))


def _trace_avgs(out_dir, sub):
    stats = [r for r in _csv_rows(os.path.join(out_dir, sub, "run_kernel_stats.csv")) if "fp8kv" in r["Name"]]
    return stats, {_short(r["Name"]): float(r["AverageNs"]) / 1e3 for r in stats}


def _counter_means(out_dir, sub, counter):
    """Mean counter value per kernel (KiB per dispatch for FETCH/WRITE_SIZE), with the copy's
    scale factor: bytes / counter of the largest device copies (2 GiB) in the same run."""
    from collections import defaultdict
    vals = defaultdict(list)
    for r in _csv_rows(os.path.join(out_dir, sub, "run_counter_collection.csv")):
        if r["Counter_Name"] == counter:
            vals[_short(r["Kernel_Name"])].append(float(r["Counter_Value"]))
    copy = [v for k, vs in vals.items() if "copyBuffer" in k for v in vs]
    big = [v for v in copy if v >= 0.9 * max(copy)]
    factor = COPY_BYTES / (sum(big) / len(big) * 1024.0)
    return {k: (sum(v) / len(v), len(v)) for k, v in vals.items()}, factor, len(big)


def summarize_profiles(out_dir: str) -> None:
    """Write the committed text summaries from the rocprofv3 runs in PROFILE_CMDS
    (run from the repository root, OUT = out_dir); each summary is written only
    if its runs are present."""
    for wl in WORKLOADS:
        if os.path.isdir(os.path.join(out_dir, f"trace_{wl}")):
            summarize_workload_trace(out_dir, wl)
        if os.path.isdir(os.path.join(out_dir, f"pmc_fetch_{wl}")) and \
                os.path.isdir(os.path.join(out_dir, f"pmc_write_{wl}")):
            summarize_workload_counters(out_dir, wl)
    if os.path.isdir(os.path.join(out_dir, "trace_next")):
        summarize_next(out_dir)
    if os.path.isdir(os.path.join(out_dir, "pmc_sq")) and os.path.isdir(os.path.join(out_dir, "pmc_tcc")):
        summarize_sq_tcc(out_dir)


def summarize_workload_trace(out_dir: str, wl: str) -> None:
    """Kernel times of bench.py --workload wl --decode-only (both KV dtypes), and one step's
    kernels: append + page check, decode, merge."""
    stats, avg = _trace_avgs(out_dir, f"trace_{wl}")
    path = os.path.join(ROOT, "profiles", f"decode_kernel_{wl}_trace.md")
    lines = [f"# Kernel trace of bench.py on the {wl} workload (FP8 and BF16 KV, decode legs only)", "",
             WORKLOADS[wl][0] + ".", "",
             "Command (from the repository root; OUT is any output folder):", "",
             f"    export TMPDIR=/tmp && {PROFILE_CMDS['trace_wl'].format(wl=wl)}", "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        name = _short(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {avg[name]:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    mrg = [k for k in avg if k.startswith("merge_kernel")]
    for kv, kv_name in ((0, "FP8"), (1, "BF16")):
        dec, app = DECODE_KERNEL[kv], f"append_check_kernel<{kv}>"
        if dec in avg and app in avg and mrg:
            m = avg[mrg[0]]
            lines += ["", f"One {kv_name} step (paged_decode_step, tags on) = `{app}` + `{dec}` + `{mrg[0]}` = "
                          f"{avg[app]:.2f} + {avg[dec]:.2f} + {m:.2f} = {avg[app] + avg[dec] + m:.2f} us of kernel "
                          f"time (the merge average covers both dtypes)."]
    lines += ["", "decode_kernel<0, ...> is the FP8-cache instance, <1, ...> the BF16 one; quant_append_kernel is the "
                  "bulk fill of the cache before timing; append_check_kernel is each step's append with the page "
                  "check in the same launch.  The averages include the 300 warm-up steps, whose first few run "
                  "before the GPU is back at full clock.", "",
              f"kernel_source_hash: {kernel_source_hash()}", ""]
    with open(path, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {path}")


def summarize_workload_counters(out_dir: str, wl: str) -> None:
    """HBM traffic of each step kernel per launch, per KV dtype, from FETCH_SIZE and WRITE_SIZE
    passes, against the algorithmic bytes the same run reported (line.json)."""
    fetch, ff, nc = _counter_means(out_dir, f"pmc_fetch_{wl}", "FETCH_SIZE")
    write, wf, _ = _counter_means(out_dir, f"pmc_write_{wl}", "WRITE_SIZE")
    with open(os.path.join(out_dir, f"pmc_fetch_{wl}", "line.json")) as f:
        line = json.loads(f.read())
    for kv, kv_name in ((0, "fp8"), (1, "bf16")):
        dec = DECODE_KERNEL[kv]
        if dec not in fetch or dec not in write or kv_name not in line.get("legs", {}):
            continue
        leg = line["legs"][kv_name]
        app = f"append_check_kernel<{kv}>"
        mrg = next((k for k in fetch if k.startswith("merge_kernel")), None)
        dec_bytes = fetch[dec][0] * 1024.0 * ff + write[dec][0] * 1024.0 * wf
        step_bytes = dec_bytes
        for k in (app, mrg):
            if k in fetch and k in write:
                step_bytes += fetch[k][0] * 1024.0 * ff + write[k][0] * 1024.0 * wf
        out = [
            f"# HBM traffic of the {kv_name.upper()} decode kernel ({dec}) and of the whole step",
            f"# (append_check_kernel<{kv}> + decode + merge) on the {wl} workload, per launch, from two",
            "# rocprofv3 counter passes (from the repository root; OUT is any folder):",
            "#   export TMPDIR=/tmp && " + PROFILE_CMDS["fetch_wl"].format(wl=wl),
            "#   export TMPDIR=/tmp && " + PROFILE_CMDS["write_wl"].format(wl=wl),
            "# Counters are KiB per dispatch; each is scaled by bytes / counter of the 2 GiB device copy",
            "# (__amd_rocclr_copyBuffer) that bench.py runs in the same process.  The merge kernel's figures",
            "# average both dtypes' calls.  Algorithmic bytes come from the same run's JSON line.",
            f"kernel_source_hash: {kernel_source_hash()}",
            f"decode_dispatches: {fetch[dec][1]}",
            f"copy_dispatches: {nc}",
            f"fetch_kib_per_dispatch_decode: {fetch[dec][0]:.1f}",
            f"write_kib_per_dispatch_decode: {write[dec][0]:.1f}",
        ]
        for label, k in (("append_check", app), ("merge", mrg)):
            if k in fetch and k in write:
                out += [f"fetch_kib_per_dispatch_{label}: {fetch[k][0]:.1f}",
                        f"write_kib_per_dispatch_{label}: {write[k][0]:.1f}"]
        out += [
            f"fetch_scale: {ff:.4f}",
            f"write_scale: {wf:.4f}",
            f"decode_traffic_bytes_per_launch: {dec_bytes:.0f}",
            f"decode_algorithmic_bytes_per_launch: {leg['alg_bytes_decode']}",
            f"decode_traffic_over_algorithmic: {dec_bytes / leg['alg_bytes_decode']:.4f}",
            f"step_traffic_bytes: {step_bytes:.0f}",
            f"step_algorithmic_bytes: {leg['alg_bytes_step']}",
            f"step_traffic_over_algorithmic: {step_bytes / leg['alg_bytes_step']:.4f}",
            "",
        ]
        path = counters_path(wl, kv_name)
        with open(path, "w") as f:
            f.write("\n".join(out))
        print(f"wrote {path}")


def summarize_next(out_dir: str) -> None:
    """Kernel times of the NEXT legs (page pool, hand-off, INT4 GEMV), and the INT4 GEMV's traffic."""
    stats, avg = _trace_avgs(out_dir, "trace_next")
    lines = ["# Kernel trace of bench.py --next-only: page pool, prefill hand-off and INT4 GEMV legs", "",
             "Command (from the repository root; OUT is any output folder):", "",
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["trace_next"], "",
             "| kernel | calls | average us | min us | max us |", "|---|---|---|---|---|"]
    for r in stats:
        name = _short(r["Name"])
        lines.append(f"| `{name}` | {r['Calls']} | {avg[name]:.2f} | {float(r['MinNs']) / 1e3:.2f} | "
                     f"{float(r['MaxNs']) / 1e3:.2f} |")
    lines += ["", f"kernel_source_hash: {kernel_source_hash(INT4_SOURCES)} (int4_gemv.hip, common.hpp)", ""]
    with open(PROFILE_NEXT, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {PROFILE_NEXT}")
    if not (os.path.isdir(os.path.join(out_dir, "pmc_fetch_next")) and
            os.path.isdir(os.path.join(out_dir, "pmc_write_next"))):
        return
    fetch, ff, _ = _counter_means(out_dir, "pmc_fetch_next", "FETCH_SIZE")
    write, wf, _ = _counter_means(out_dir, "pmc_write_next", "WRITE_SIZE")
    n_, k_ = 28672, 8192
    lines = ["# INT4 weight-only GEMV on a 28672 x 8192 projection (bench.py's int4_gemv leg)", "",
             "Commands (from the repository root; OUT is any output folder):", "",
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["trace_next"],
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["fetch_next"],
             "    export TMPDIR=/tmp && " + PROFILE_CMDS["write_next"], "",
             "Average kernel time from the trace; FETCH_SIZE / WRITE_SIZE (KiB per dispatch) scaled by the "
             f"2 GiB device copy's factors ({ff:.4f} / {wf:.4f}); algorithmic bytes = codes n*k/2 + scales "
             "n*k/64 + x 2*m*k + y 2*m*n.", "",
             "| M | kernel | average us | algorithmic MB | HBM MB (fetch + write) | traffic / algorithmic | "
             "GB/s (algorithmic / average) | % of 8 TB/s |",
             "|---|---|---|---|---|---|---|---|"]
    for m_, kname in INT4_INSTANCES.items():
        if kname not in avg or kname not in fetch or kname not in write:
            continue
        alg4 = n_ * k_ // 2 + n_ * (k_ // 128) * 2 + 2 * m_ * k_ + 2 * m_ * n_
        hbm = (fetch[kname][0] * ff + write[kname][0] * wf) * 1024.0
        gbps = alg4 / (avg[kname] * 1e-6) / 1e9
        lines.append(f"| {m_} | `{kname}` | {avg[kname]:.2f} | {alg4 / 1e6:.1f} | {hbm / 1e6:.1f} | "
                     f"{hbm / alg4:.3f} | {gbps:.0f} | {100 * gbps / PEAK_HBM_GBPS:.1f} |")
    lines += ["", f"kernel_source_hash: {kernel_source_hash(INT4_SOURCES)} (int4_gemv.hip, common.hpp)", ""]
    with open(PROFILE_INT4, "w") as f:
        f.write("\n".join(lines))
    print(f"wrote {PROFILE_INT4}")


def summarize_sq_tcc(out_dir: str) -> None:
    """Instruction mix, LDS conflicts and L2 hit rate of the FP8 decode kernel (per dispatch), headline workload."""
    from collections import defaultdict
    vals = defaultdict(lambda: defaultdict(float))
    for sub_dir in ("pmc_sq", "pmc_tcc", "pmc_lds"):
        if not os.path.isdir(os.path.join(out_dir, sub_dir)):
            continue
        for r in _csv_rows(os.path.join(out_dir, sub_dir, "run_counter_collection.csv")):
            if _short(r["Kernel_Name"]) == DECODE_KERNEL[0]:
                vals[r["Counter_Name"]][(sub_dir, r["Dispatch_Id"])] += float(r["Counter_Value"])
    avg = {k: sum(d.values()) / len(d) for k, d in vals.items() if d}
    from decode_attention_fp8_kv_amd import workloads as W
    w = W.make(WORKLOAD)
    tiles = sum(-(-int(L) // 64) for L in w.seq_lens) * w.num_kv_heads   # upper bound: aborted ones included
    out = [f"# {DECODE_KERNEL[0]} (FP8 cache) on the {WORKLOAD} workload: instruction mix, LDS bank",
           "# conflicts and L2 hits, per dispatch, from three rocprofv3 counter passes (repository root; OUT any folder):",
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["sq"],
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["tcc"],
           "#   export TMPDIR=/tmp && " + PROFILE_CMDS["lds"],
           "# (a counter read in two passes is averaged over both; SQ_LDS_BANK_CONFLICT, in cycles, has a pass",
           "# of its own; it equals SQ_INSTS_MFMA here because both come to 32 per tile)",
           f"kernel_source_hash: {kernel_source_hash()}"]
    for k in sorted(avg):
        out.append(f"{k}: {avg[k]:.0f}")
    if avg.get("SQ_INSTS_LDS") and "SQ_LDS_BANK_CONFLICT" in avg:
        out.append(f"lds_bank_conflict_cycles_per_lds_instruction: "
                   f"{avg['SQ_LDS_BANK_CONFLICT'] / avg['SQ_INSTS_LDS']:.3f}")
    tiles_ok = avg.get("SQ_INSTS_MFMA", 0.0) / 32.0   # 32 MFMAs per (sequence, KV head, tile) on this path
    if tiles_ok:
        out.append(f"tiles_decoded_per_dispatch: {tiles_ok:.0f}   # SQ_INSTS_MFMA / 32")
        if "SQ_INSTS_VALU" in avg:
            out.append(f"valu_instructions_per_tile: {avg['SQ_INSTS_VALU'] / tiles_ok:.0f}")
        if "SQ_INSTS_VMEM_RD" in avg:
            out.append(f"vmem_read_instructions_per_tile: {avg['SQ_INSTS_VMEM_RD'] / tiles_ok:.1f}")
        if "SQ_INSTS_LDS" in avg:
            out.append(f"lds_instructions_per_tile: {avg['SQ_INSTS_LDS'] / tiles_ok:.1f}")
        if "SQ_LDS_BANK_CONFLICT" in avg:
            out.append(f"lds_bank_conflict_cycles_per_tile: {avg['SQ_LDS_BANK_CONFLICT'] / tiles_ok:.1f}")
    if avg.get("TCC_HIT_sum", 0) + avg.get("TCC_MISS_sum", 0) > 0:
        out.append(f"l2_hit_rate: {avg['TCC_HIT_sum'] / (avg['TCC_HIT_sum'] + avg['TCC_MISS_sum']):.4f}")
    out.append(f"# (tiles of all sequences, aborted ones included: {tiles}; the decode streams only the others)")
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
    ap.add_argument("--no-tag-ab", action="store_true", help="skip the tags on/off comparison")
    ap.add_argument("--workload", choices=sorted(WORKLOADS), default=WORKLOAD,
                    help="headline decode workload (default: conc64)")
    ap.add_argument("--decode-only", action="store_true",
                    help="only the named workload's decode legs (no other workloads, NEXT legs or CPU baseline)")
    ap.add_argument("--next-only", action="store_true", help="only the page-pool, hand-off and INT4 legs")
    ap.add_argument("--json-out", default=None, help="also write the JSON line to this file")
    args = ap.parse_args()
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) != 1:
        print("bench.py measures one GPU only: decode sequences shard across GPUs with no exchange "
              "between them, and no multi-GPU run is made.", file=sys.stderr)
        sys.exit(2)

    import torch

    import decode_attention_fp8_kv_amd as fk
    from decode_attention_fp8_kv_amd import workloads as W

    dev = torch.device("cuda:0")
    fk.load_library()
    copy_gbps = copy_bandwidth(dev)
    if args.next_only:
        line = {"page_pool": pool_timings(dev), "prefill_handoff": handoff_timings(dev),
                "int4_gemv": int4_gemv_timings(dev)}
        print(json.dumps(line), flush=True)
        return

    wl = args.workload
    tag_ab = (not args.no_tag_ab) and wl in TAG_AB_WORKLOADS
    res = run_workload(wl, dev, args.steps, args.warmup, bf16=not args.no_bf16, flushed=not args.decode_only,
                       tag_ab=tag_ab)
    f = res["fp8"]
    dec = f["decode_kernel_us"]
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
        "data": WORKLOADS[wl][1],
        "config": {
            "workload": WORKLOADS[wl][0],
            "batch": f["batch"], "num_q_heads": 64, "num_kv_heads": 8, "head_dim": 128, "page_size": 64,
            "context_tokens": f["context_tokens"], "aborted_sequences": f["aborted"], "num_pages": f["num_pages"],
            "step": "paged_decode_step: append of one token per sequence + page check (one launch), decode, merge",
            "parallelism": "single GPU",
        },
        "effective_kv_gbps": round(f["decode_gbps"], 1),
        "pct_hbm_peak": round(100.0 * f["decode_gbps"] / PEAK_HBM_GBPS, 2),
        "roofline": {
            "kernel": DECODE_KERNEL[0],
            "bound": "hbm",
            "achieved": round(f["decode_gbps"], 1),
            "peak": PEAK_HBM_GBPS,
            "unit": "GB/s",
            "frac": round(f["decode_gbps"] / PEAK_HBM_GBPS, 4),
            "traffic": f["traffic"],
            "alg_bytes_per_launch": f["alg_bytes"],
            "mean_launch_us": round(dec["mean"], 2),
            "timing": "HIP events recorded by paged_decode_step right before and right after the decode kernel, "
                      "on its launch stream, every 4th step of a sampling pass of the same length as the timed one",
        },
        "decode_kernel_us": {k: round(v, 2) for k, v in dec.items()},
        "step": {"us": {k: round(v, 2) for k, v in f["step_us"].items()}, "alg_bytes": f["alg_bytes_step"],
                 "gbps": round(f["step_gbps"], 1), "frac": round(f["step_gbps"] / PEAK_HBM_GBPS, 4),
                 "wall_frac": round(f["wall_gbps"] / PEAK_HBM_GBPS, 4)},
        "bulk_fill": f["fill"],
        "device_copy_gbps": round(copy_gbps, 1),
        "legs": {name: summary(r) for name, r in res.items()},
    }
    if "flushed" in f:
        line["step_us_flushed"] = {"median": f["flushed"][0], "p95": f["flushed"][1],
                                   "protocol": "1 GiB read before each step (evicts the Infinity Cache), "
                                               "outside the timed region; 30 steps"}
    if "bf16" in res:
        b = res["bf16"]
        line["bf16"] = {"value": round(b["value"], 1), "unit": "tokens/s", "ms_per_step": round(b["ms_per_step"], 4),
                        "batch": b["batch"], "aborted": b["aborted"],
                        "pool": ("the same bytes as the FP8 pool, sequences admitted in order while they fit"
                                 if wl == "conc64" else "the same workload"),
                        "decode_kernel_gbps": round(b["decode_gbps"], 1),
                        "decode_kernel_frac": round(b["decode_gbps"] / PEAK_HBM_GBPS, 4),
                        "decode_kernel_us": round(b["decode_kernel_us"]["mean"], 2)}
        line["fp8_over_bf16_tokens_per_s"] = round(f["value"] / b["value"], 3)
    if "tag_check" in f:
        line["tag_check"] = {wl: f["tag_check"]}
    if not args.decode_only:
        extra, tags = {}, {}
        for xw in EXTRA_WORKLOADS:
            if xw == wl:
                continue
            r = run_workload(xw, dev, args.steps, args.warmup, bf16=not args.no_bf16,
                             tag_ab=(not args.no_tag_ab) and xw in TAG_AB_WORKLOADS)
            extra[xw] = {name: summary(x) for name, x in r.items()}
            if "tag_check" in r["fp8"]:
                tags[xw] = r["fp8"]["tag_check"]
        line["workloads"] = extra
        if tags:
            line.setdefault("tag_check", {}).update(tags)
        line["page_pool"] = pool_timings(dev)
        line["prefill_handoff"] = handoff_timings(dev)
        line["int4_gemv"] = int4_gemv_timings(dev)
    if not args.no_cpu_baseline and not args.decode_only:
        line["cpu_baseline"] = cpu_baseline(W.make(wl))
    text = json.dumps(line)
    if args.json_out:
        os.makedirs(os.path.dirname(os.path.abspath(args.json_out)), exist_ok=True)
        with open(args.json_out, "w") as fh:
            fh.write(text + "\n")
    print(text, flush=True)


if __name__ == "__main__":
    main()
