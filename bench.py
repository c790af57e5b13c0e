#!/usr/bin/env python3
"""Benchmark of multi-row verify attention over a paged E4M3 KV cache.

One step = one verify call (split partials) + one combine call on the
headline workload: q8 rows, 6 query heads over 1 KV head, head dim 256,
E4M3 pages, context 262144 in 3456-token pages, rows 5-7 zero-length, NaN
null page padding the table (the largest configuration of the 8K-256K range
the metric is quoted on).  The KV pool is replicated in device memory and the
steps rotate through the copies, so every call reads K/V from HBM rather than
from the 256 MB Infinity Cache ("cold"); the same loop on one copy ("hot",
identical inputs back to back) is reported beside it, with the other contexts
of the range (8K, 64K, 128K) and the sparse (QSA) batch.

Per-call time is measured on a HIP graph of consecutive verify + combine calls,
replayed (the pages time their kernels from CUDA-graph samples), so that Python
launch overhead does not set the pace: exactly --steps calls are timed, and the
percentiles come from a separate sample of 60 replays; the eager per-call time
is reported beside it.  Throughput counts algorithmic bytes only: the longest
visible prefix x 512 B (K and V, one KV head, D = 256, one byte per element).
The verify kernel's own duration comes from the library's kernel timer (HIP
events passed with each verify dispatch, on the stream it runs on) over an
eager loop of the same calls, and roofline.achieved = algorithmic bytes / that
duration.  A plain streaming-read kernel over a 2 GiB buffer gives the
device's practical read ceiling beside the published peak.  The FP64 CPU
oracle is timed on the host's cores on the same workload as a reported
baseline.

Prints ONE JSON line on stdout; progress goes to stderr.  With --workload
naming a sparse or batch workload (c4, c4tok, batch) the line holds that
workload's timings alone ("workload_only"): the form the counter runs take.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import statistics
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

METRIC = "µs/call and KV-read GB/s (% HBM peak), q8 H6/Hkv1/D256 E4M3, 8K–256K ctx"
HBM_PEAK_GBS = 8000.0          # MI355X HBM3E, published
MALL_BYTES = 256 << 20         # Infinity Cache
PMC_FILE = os.path.join(ROOT, "profiles", "verify_kernel_pmc.json")
KERNEL_SOURCES = ("verify_mfma.hip", "pa_verify.h")


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_hash() -> str:
    """Hash of the verify kernel's sources (the kernel the counters describe)."""
    h = hashlib.sha256()
    for name in KERNEL_SOURCES:
        with open(os.path.join(ROOT, "fp8_kv_paged_attn_amd", "csrc", name), "rb") as f:
            h.update(name.encode() + b"\0" + f.read())
    return h.hexdigest()[:16]


class DenseBench:
    """A dense workload resident on the device, with n_copies of its KV pool."""

    def __init__(self, w, n_copies: int, kernel: str, splits: int):
        import numpy as np
        import torch

        import fp8_kv_paged_attn_amd as pa

        self.w, self.pa, self.torch = w, pa, torch
        dev = torch.device("cuda:0")
        self.q = torch.from_numpy(np.ascontiguousarray(w.q_bits).view(np.int16)).view(
            torch.float16).to(dev)
        k = torch.from_numpy(w.k_pool).to(dev)
        v = torch.from_numpy(w.v_pool).to(dev)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n_copies - 1)]
        self.table = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)
        self.lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(dev)
        G = w.num_heads // w.num_kv_heads
        s = splits if splits else w.num_splits
        self.plan = pa.plan(w.max_tokens, w.q_rows * G, w.num_kv_heads, w.head_dim, w.page_size,
                            splits=s, kernel=kernel)
        self.rows = w.q_rows * w.num_heads
        self.ws = pa.make_workspace(self.plan, self.rows, w.head_dim, dev)
        self.out = torch.empty((w.q_rows, w.num_heads, w.head_dim), dtype=torch.float16,
                               device=dev)
        self.kv_bytes = w.kv_bytes()
        self.pool_bytes = 2 * k.numel()

    def verify(self, i: int):
        k, v = self.pools[i % len(self.pools)]
        w = self.w
        self.pa.paged_attn_verify_e4m3(self.q, k, v, self.table, self.lens, w.max_tokens,
                                       w.sm_scale, w.k_scale, self.plan, self.ws)

    def combine(self):
        self.pa.paged_attn_combine_fp32(self.ws, self.plan.num_splits, self.rows,
                                        self.w.head_dim, self.w.v_scale, self.out)

    def combine_lse(self, out32, lse):
        self.pa.paged_attn_combine_fp32_lse(self.ws, self.plan.num_splits, self.rows,
                                            self.w.head_dim, self.w.v_scale, out32=out32,
                                            lse=lse)

    def time_combines(self, reps: int = 20) -> dict:
        """Combines over the workspace of the last verify (so the partials are
        in cache), from graph replays of GRAPH_CALLS back-to-back launches: FP16
        output, and FP32 output + base-2 LSE."""
        torch = self.torch
        D = self.w.head_dim
        out32 = torch.empty(self.rows * D, dtype=torch.float32, device="cuda:0")
        lse = torch.empty(self.rows, dtype=torch.float32, device="cuda:0")
        res = {}
        fns = [("combine_us", self.combine)]
        if self.plan.selection != self.pa.PA_SELECTION["batch"]:
            fns.append(("combine_lse_us", lambda: self.combine_lse(out32, lse)))
        for name, fn in fns:
            side = torch.cuda.Stream()
            side.wait_stream(torch.cuda.current_stream())
            with torch.cuda.stream(side):
                fn()
            torch.cuda.current_stream().wait_stream(side)
            torch.cuda.synchronize()
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for _ in range(GRAPH_CALLS):
                    fn()
            g.replay()
            torch.cuda.synchronize()
            e0 = torch.cuda.Event(enable_timing=True)
            e1 = torch.cuda.Event(enable_timing=True)
            e0.record()
            for _ in range(reps):
                g.replay()
            e1.record()
            torch.cuda.synchronize()
            res[name] = round(e0.elapsed_time(e1) * 1e3 / (reps * GRAPH_CALLS), 3)
            del g
        S = self.plan.num_splits
        res["workspace_bytes"] = S * self.rows * (D + 2) * 4
        res["timing"] = f"{reps} replays of a graph of {GRAPH_CALLS} launches"
        return res

    def run_graph(self, steps: int, warmup: int, rotate: bool):
        """Per-call time of verify + combine replayed from HIP graphs.

        Graphs of c = gcd(steps, GRAPH_CALLS) consecutive calls are captured
        once: one on the first pool copy, or (rotate) enough of them that their
        calls read every pool copy in turn.  After at least `warmup` untimed
        calls, exactly `steps` calls (steps / c replays, cycling through the
        graphs) are timed between two synchronisations; that gives ms per call.
        A separate sample of PCT_REPLAYS replays, an event after each, sets
        self.pcts (the per-call percentiles), so that they rest on at least 50
        samples whatever `steps` is."""
        torch = self.torch
        calls = math.gcd(max(1, steps), GRAPH_CALLS)
        # rotating: graph q holds the calls on copies q*calls .. q*calls + calls - 1
        # (mod the copy count), and the replays cycle through the graphs, so
        # that consecutive calls read every copy in turn
        ngraphs = -(-len(self.pools) // calls) if rotate else 1
        copy = lambda q, i: (q * calls + i) % len(self.pools) if rotate else 0
        side = torch.cuda.Stream()
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            for i in range(calls):
                self.verify(copy(0, i))
                self.combine()
        torch.cuda.current_stream().wait_stream(side)
        torch.cuda.synchronize()
        graphs = []
        for q in range(ngraphs):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(calls):
                    self.verify(copy(q, i))
                    self.combine()
            graphs.append(g)
        torch.cuda.synchronize()
        for r in range(max(ngraphs, -(-warmup // calls))):
            graphs[r % ngraphs].replay()
        torch.cuda.synchronize()
        reps = max(1, steps // calls)
        e0 = torch.cuda.Event(enable_timing=True)
        e1 = torch.cuda.Event(enable_timing=True)
        e0.record()
        for r in range(reps):
            graphs[r % ngraphs].replay()
        e1.record()
        torch.cuda.synchronize()
        total_ms = e0.elapsed_time(e1)
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(PCT_REPLAYS + 1)]
        marks[0].record()
        for k in range(PCT_REPLAYS):
            graphs[k % ngraphs].replay()
            marks[k + 1].record()
        torch.cuda.synchronize()
        self.pcts = percentiles([marks[k].elapsed_time(marks[k + 1]) / calls
                                 for k in range(PCT_REPLAYS)], calls)
        del graphs
        return total_ms / (reps * calls)

    def output(self):
        """One verify + combine on the first pool copy, as float64 on the host."""
        self.verify(0)
        self.combine()
        self.torch.cuda.synchronize()
        return self.out.float().cpu().numpy().astype("float64").reshape(self.out.shape)

    def run(self, steps: int, warmup: int, rotate: bool):
        """Time `steps` eager calls; returns (ms per call, mean and median verify-kernel ms).

        The timed region holds the calls alone.  Each verify kernel's own run
        is timed by the library's kernel timer (HIP events bound to the
        dispatch), which adds no commands to the stream."""
        torch, pa = self.torch, self.pa
        for i in range(warmup):
            self.verify(i if rotate else 0)
            self.combine()
        torch.cuda.synchronize()
        # an event every SAMPLE calls: per-call percentiles over the samples
        marks = [torch.cuda.Event(enable_timing=True) for _ in range(steps // SAMPLE + 2)]
        pa.timer_arm(min(steps, pa.TIMER_MAX_LAUNCHES))
        marks[0].record()
        nm = 1
        for i in range(steps):
            self.verify(i if rotate else 0)
            self.combine()
            if (i + 1) % SAMPLE == 0 or i + 1 == steps:
                marks[nm].record()
                nm += 1
        torch.cuda.synchronize()
        total_ms = marks[0].elapsed_time(marks[nm - 1])
        per_call = [marks[k - 1].elapsed_time(marks[k]) / SAMPLE
                    for k in range(1, nm) if k * SAMPLE <= steps]
        self.pcts = percentiles(per_call, SAMPLE)
        vk = pa.timer_read()
        return total_ms / steps, statistics.fmean(vk), statistics.median(vk)


SAMPLE = 10          # eager calls per timing sample
GRAPH_CALLS = 10     # verify + combine calls captured in one graph (at most)
PCT_REPLAYS = 60     # graph replays behind the per-call percentiles


def percentiles(xs, calls_per_sample: int):
    """p10/p50/p90, mean and max (us) of per-call times given in ms."""
    if not xs:
        return None
    ys = sorted(x * 1e3 for x in xs)
    pick = lambda q: ys[min(len(ys) - 1, int(round(q * (len(ys) - 1))))]
    return {"p10": round(pick(0.1), 3), "p50": round(pick(0.5), 3), "p90": round(pick(0.9), 3),
            "mean": round(sum(ys) / len(ys), 3), "max": round(ys[-1], 3),
            "samples": len(ys), "calls_per_sample": calls_per_sample}


class QsaBench(DenseBench):
    """The sparse (QSA) batch resident on the device, with n_copies of its pool."""

    def __init__(self, w, n_copies: int, kernel: str):
        self._setup(w, n_copies, w.sel_blocks, w.topk * w.page_size, "blocks", kernel)

    def _setup(self, w, n_copies: int, sel, list_len: int, selection: str, kernel: str):
        import numpy as np
        import torch

        import fp8_kv_paged_attn_amd as pa

        self.w, self.pa, self.torch = w, pa, torch
        dev = torch.device("cuda:0")
        self.q = torch.from_numpy(np.ascontiguousarray(w.q_bits).view(np.int16)).view(
            torch.bfloat16).to(dev)
        k = torch.from_numpy(w.k_pool).to(dev)
        v = torch.from_numpy(w.v_pool).to(dev)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n_copies - 1)]
        self.table = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)
        self.sel = torch.from_numpy(sel.astype(np.int32)).to(dev)
        self.lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(dev)
        G = w.num_heads // w.num_kv_heads
        self.plan = pa.plan(list_len, w.q_rows * G, w.batch * w.num_kv_heads, w.head_dim,
                            w.page_size, selection, splits=w.num_splits, kernel=kernel)
        self.rows = w.num_rows
        self.ws = pa.make_workspace(self.plan, self.rows, w.head_dim, dev)
        self.out = torch.empty((w.batch, w.q_rows, w.num_heads, w.head_dim),
                               dtype=torch.float16, device=dev)
        self.kv_bytes = w.kv_bytes()

    def verify(self, i: int):
        k, v = self.pools[i % len(self.pools)]
        w = self.w
        self.pa.qsa_sparse_verify_e4m3(self.q, k, v, self.table, self.sel, self.lens, w.sm_scale,
                                       w.k_scale, self.plan, self.ws)


class QsaTokensBench(QsaBench):
    """The sparse batch over selected token ids, resident on the device."""

    def __init__(self, w, n_copies: int, kernel: str):
        self._setup(w, n_copies, w.sel_tokens, w.num_sel, "tokens", kernel)

    def verify(self, i: int):
        k, v = self.pools[i % len(self.pools)]
        w = self.w
        self.pa.qsa_sparse_verify_tokens_e4m3(self.q, k, v, self.table, self.sel, self.lens,
                                              w.sm_scale, w.k_scale, self.plan, self.ws)


def bench_for(w, kernel: str, splits: int = 0):
    """The resident bench of a named workload (dense, sparse over blocks or token
    ids, or a batch of independent requests)."""
    n = copies_for(w.kv_bytes())
    if hasattr(w, "sel_tokens"):
        return QsaTokensBench(w, n, kernel)
    if hasattr(w, "sel_blocks"):
        return QsaBench(w, n, kernel)
    if hasattr(w, "request"):
        return BatchBench(w, n, kernel)
    return DenseBench(w, n, kernel, splits)


def measure(b, steps: int, warmup: int) -> dict:
    """Cold (rotating pool copies) and hot (one copy) timings of one workload:
    per-call time from graph replays, verify-kernel time from the eager,
    timer-armed loop (in microseconds)."""
    c_ms = b.run_graph(steps, warmup, rotate=True)
    c_pcts = b.pcts
    e_ms, vk, vmed = b.run(steps, warmup, rotate=True)
    h_ms = b.run_graph(steps, warmup, rotate=False)
    h_pcts = b.pcts
    _, h_vk, _ = b.run(steps, warmup, rotate=False)
    return {"us": c_ms * 1e3, "pcts": c_pcts, "eager_us": e_ms * 1e3, "verify_us": vk * 1e3,
            "verify_med_us": vmed * 1e3, "hot_us": h_ms * 1e3, "hot_pcts": h_pcts,
            "hot_verify_us": h_vk * 1e3, "out": b.output()}


def sweep_entry(name: str, kv_bytes: int, plan, m: dict, **extra) -> dict:
    gb = lambda us: round(kv_bytes / (us * 1e-6) / 1e9, 1)
    return {"workload": name, **extra, "kv_bytes": kv_bytes, "splits": plan.num_splits,
            "tokens_per_split": plan.tokens_per_split,
            "rows_per_workgroup": plan.rows_per_workgroup,
            "us_per_call": round(m["us"], 3), "gbs": gb(m["us"]),
            "us_per_call_pcts": m["pcts"],
            "verify_us": round(m["verify_us"], 3), "verify_gbs": gb(m["verify_us"]),
            "eager_us_per_call": round(m["eager_us"], 3),
            "hot_us_per_call": round(m["hot_us"], 3), "hot_gbs": gb(m["hot_us"]),
            "hot_verify_us": round(m["hot_verify_us"], 3)}


def error_figures(gpu, ref) -> dict:
    """The GPU output against the FP64 oracle output o: rel-L2 and max-abs, with
    the FP16 output-rounding floor of o beside each (rel-L2 of fp16(o), and
    max |fp16(o) - o|), as the design note "DFlash2 E4M3 attention with FP32
    state" reports its errors ("Observability and reproduction")."""
    import numpy as np

    gpu = np.asarray(gpu, np.float64).ravel()
    ref = np.asarray(ref, np.float64).ravel()
    fin = np.isfinite(ref)
    if not np.array_equal(np.isfinite(gpu), fin):
        return {"finite_pattern_matches": False}
    g, o = gpu[fin], ref[fin]
    r16 = o.astype(np.float16).astype(np.float64)
    norm = float(np.linalg.norm(o)) or 1.0
    return {"rel_l2": float(f"{np.linalg.norm(g - o) / norm:.4e}"),
            "floor_rel_l2": float(f"{np.linalg.norm(r16 - o) / norm:.4e}"),
            "max_abs": float(f"{np.abs(g - o).max(initial=0.0):.4e}"),
            "floor_abs": float(f"{np.abs(r16 - o).max(initial=0.0):.4e}")}


def oracle_output(orc, w, threads: int):
    """The FP64 oracle's output for any of the bench workloads."""
    import numpy as np

    if hasattr(w, "sel_tokens"):
        return orc.qsa_tokens_workload(w, nthreads=threads)
    if hasattr(w, "sel_blocks"):
        return orc.qsa_workload(w, nthreads=threads)
    if hasattr(w, "request"):
        return np.stack([orc.dense_workload(w.request(b), nthreads=threads)
                         for b in range(w.batch)])
    return orc.dense_workload(w, nthreads=threads)


class BatchBench(DenseBench):
    """A batch of independent dense requests resident on the device."""

    def __init__(self, w, n_copies: int, kernel: str):
        import numpy as np
        import torch

        import fp8_kv_paged_attn_amd as pa

        self.w, self.pa, self.torch = w, pa, torch
        dev = torch.device("cuda:0")
        self.q = torch.from_numpy(np.ascontiguousarray(w.q_bits).view(np.int16)).view(
            torch.float16).to(dev)
        k = torch.from_numpy(w.k_pool).to(dev)
        v = torch.from_numpy(w.v_pool).to(dev)
        self.pools = [(k, v)] + [(k.clone(), v.clone()) for _ in range(n_copies - 1)]
        self.table = torch.from_numpy(w.block_table.astype(np.int32)).to(dev)
        self.lens = torch.from_numpy(w.row_lens.astype(np.int32)).to(dev)
        G = w.num_heads // w.num_kv_heads
        # one ragged split plan over the whole batch: the splits are shared out
        # over the requests in proportion to their lengths
        self.plan = pa.plan(w.cap, w.q_rows * G, w.batch * w.num_kv_heads, w.head_dim,
                            w.page_size, "batch", splits=w.num_splits, kernel=kernel)
        self.rows = w.num_rows
        self.ws = pa.make_workspace(self.plan, self.rows, w.head_dim, dev)
        self.out = torch.empty((w.batch, w.q_rows, w.num_heads, w.head_dim),
                               dtype=torch.float16, device=dev)
        self.kv_bytes = w.kv_bytes()

    def verify(self, i: int):
        k, v = self.pools[i % len(self.pools)]
        w = self.w
        self.pa.paged_attn_verify_batch_e4m3(self.q, k, v, self.table, self.lens, w.sm_scale,
                                             w.k_scale, self.plan, self.ws)

    def combine(self):
        w = self.w
        self.pa.paged_attn_combine_batch_fp32(self.ws, self.plan, w.batch, w.q_rows, w.num_heads,
                                              w.num_kv_heads, w.head_dim, w.v_scale, self.out)


def time_cache_write(torch, pa, tokens: int, reps: int = 20) -> dict:
    """E4M3 cache write of `tokens` FP16 K/V tokens (H1, D256, pages of 3456) into
    shuffled slots, from graph replays of GRAPH_CALLS writes."""
    D, ps = 256, 3456
    pages = -(-tokens // ps) + 1
    g = torch.Generator(device="cpu").manual_seed(0xCAC4E)
    k = torch.randn((tokens, 1, D), generator=g).to(torch.float16).to("cuda:0")
    v = torch.randn((tokens, 1, D), generator=g).to(torch.float16).to("cuda:0")
    slots = torch.randperm(pages * ps, generator=g)[:tokens].to(torch.int64).to("cuda:0")
    kp = torch.zeros((pages, ps, 1, D), dtype=torch.uint8, device="cuda:0")
    vp = torch.zeros_like(kp)
    fn = lambda: pa.paged_attn_cache_write_e4m3(k, v, slots, kp, vp, 0.5, 2.0)
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        for _ in range(GRAPH_CALLS):
            fn()
    graph.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        graph.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * GRAPH_CALLS)
    nbytes = tokens * D * (2 * 2 + 2 * 1)          # FP16 K, V read; E4M3 K, V written
    del graph
    return {"tokens": tokens, "us": round(us, 3), "bytes": nbytes,
            "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def read_ceiling(torch, pa, nbytes: int = 2 << 30, reps: int = 5):
    """Read bandwidth (GB/s) of the plain streaming-read probe over nbytes."""
    buf = torch.zeros(nbytes // 16, 4, dtype=torch.int32, device="cuda:0")
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    for _ in range(2):
        pa.stream_read_probe(buf, sink)
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        pa.stream_read_probe(buf, sink)
    e1.record()
    torch.cuda.synchronize()
    gbs = nbytes * reps / (e0.elapsed_time(e1) * 1e-3) / 1e9
    del buf
    torch.cuda.empty_cache()
    return round(gbs, 1)


def read_ceiling_at(torch, pa, nbytes: int, reps: int = 20) -> dict:
    """The streaming-read probe over nbytes, cold like the verify timing
    (rotating over enough buffers that one rotation exceeds twice the Infinity
    Cache), timed from graph replays of GRAPH_CALLS probe launches: the best a
    plain read kernel does on the same number of bytes."""
    ncop = copies_for(nbytes)
    bufs = [torch.zeros(nbytes // 16, 4, dtype=torch.int32, device="cuda:0") for _ in range(ncop)]
    sink = torch.zeros(1, dtype=torch.int32, device="cuda:0")
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        for i in range(GRAPH_CALLS):
            pa.stream_read_probe(bufs[i % ncop], sink)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        for i in range(GRAPH_CALLS):
            pa.stream_read_probe(bufs[i % ncop], sink)
    for _ in range(3):
        g.replay()
    torch.cuda.synchronize()
    e0 = torch.cuda.Event(enable_timing=True)
    e1 = torch.cuda.Event(enable_timing=True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / (reps * GRAPH_CALLS)
    del g, bufs
    torch.cuda.empty_cache()
    return {"bytes": nbytes, "us": round(us, 3), "gbs": round(nbytes / (us * 1e-6) / 1e9, 1)}


def copies_for(touched_bytes: int) -> int:
    """Enough pool copies that the bytes one rotation reads (touched_bytes per
    call) exceed twice the Infinity Cache."""
    return max(2, math.ceil(2 * MALL_BYTES / max(touched_bytes, 1)) + 1)


def cpu_baseline(w, outputs: dict, max_seconds: float = 20.0):
    """The FP64 oracle timed on the host on the headline workload, and run once
    on every workload the bench measured, whose outputs (`outputs`: name ->
    (workload, GPU output)) it is compared with (the accuracy figures).

    Threads: the CPUs this process may use, at most 16 (a host's share of CPUs
    per GPU on an 8-GPU MI355X node); the host's CPU count is reported beside it."""
    import oracle

    orc = oracle.get()
    avail = len(os.sched_getaffinity(0)) if hasattr(os, "sched_getaffinity") else (os.cpu_count() or 1)
    threads = max(1, min(16, avail))
    times = []
    t_start = time.perf_counter()
    ref = None
    while len(times) < 3 and (time.perf_counter() - t_start) < max_seconds:
        t0 = time.perf_counter()
        ref = orc.dense_workload(w, nthreads=threads)
        times.append(time.perf_counter() - t0)
    t = statistics.median(times)
    t0 = time.perf_counter()
    orc.dense_workload(w, nthreads=1)
    t1 = time.perf_counter() - t0
    accuracy = {}
    for name, (wk, gpu) in outputs.items():
        o = ref if name == w.name else oracle_output(orc, wk, threads)
        accuracy[name] = error_figures(gpu, o)
    return {"value": round(w.kv_bytes() / t / 1e9, 4), "unit": "GB/s", "cores": threads,
            "kind": "oracle",
            "sample": f"the whole {w.name} workload (all {w.q_rows} rows x {w.num_heads} heads), "
                      f"FP64 oracle on {threads} threads, median of {len(times)} runs, "
                      f"{t * 1e3:.1f} ms per call",
            "host_cpus": os.cpu_count(), "cpus_available": avail,
            "value_1thread": round(w.kv_bytes() / t1 / 1e9, 4),
            "sample_1thread": f"the same workload on 1 thread, one run, {t1 * 1e3:.1f} ms"}, \
        accuracy


def traffic_from_profile(src_hash: str, workload: str):
    """HBM bytes per verify launch for `workload` from the committed counter runs
    (FETCH_SIZE and WRITE_SIZE scaled by the copy calibration), or None when the
    kernel sources have changed since the counters were taken."""
    try:
        with open(PMC_FILE) as f:
            d = json.load(f)
    except (OSError, ValueError):
        return None
    if d.get("source_hash") != src_hash:
        return None
    return d.get("workloads", {}).get(workload, {}).get("hbm_bytes_per_launch")


def main():
    ap = argparse.ArgumentParser(description=__doc__.split("\n")[0])
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=200)
    ap.add_argument("--warmup", type=int, default=400)
    ap.add_argument("--workload", default="c3")
    ap.add_argument("--kernel", default="mfma", choices=["auto", "simple", "mfma"])
    ap.add_argument("--splits", type=int, default=0)
    ap.add_argument("--no-sweep", action="store_true")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--copy-probe", type=int, default=0, metavar="MIB",
                    help="also run one plain device-to-device copy of MIB MiB (a known-size "
                         "kernel for calibrating hardware traffic counters) before the benchmark")
    args = ap.parse_args()

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this benchmark runs on one GPU only; the verify path is "
                                   "measured on a single MI355X (--gpus 1)",
                          "n_gpus": args.gpus}))
        sys.exit(2)

    import torch

    import fp8_kv_paged_attn_amd as pa
    from fp8_kv_paged_attn_amd import workloads as wl

    if not torch.cuda.is_available():
        raise SystemExit("bench.py needs a ROCm GPU (cuda:0)")
    pa.lib()
    src_hash = kernel_source_hash()

    if args.copy_probe:
        n = args.copy_probe << 20
        src = torch.empty(n, dtype=torch.uint8, device="cuda:0").fill_(1)
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        log(f"[bench] copy probe: {n} bytes read, {n} bytes written")

    log(f"[bench] generating {args.workload}")
    w = wl.cached(args.workload)
    n_copies = copies_for(w.kv_bytes())
    log(f"[bench] {w.name}: {n_copies} pool copies, kernel={args.kernel}")
    b = bench_for(w, args.kernel, args.splits)
    if not isinstance(w, wl.DenseWorkload):
        # a sparse or batch workload on its own (counter and trace runs): its
        # timings, without the headline record, which is a dense figure
        m = measure(b, args.steps, args.warmup)
        m.pop("out")
        e = sweep_entry(w.name, b.kv_bytes, b.plan, m, units=w.batch * w.num_kv_heads)
        e["traffic"] = traffic_from_profile(src_hash, w.name)
        print(json.dumps({"workload_only": e, "source_hash": src_hash,
                          "build_id": pa.build_id()}), flush=True)
        return
    m = measure(b, args.steps, args.warmup)
    log(f"[bench] cold: {m['us']:.2f} us/call (graph), {m['eager_us']:.2f} eager, "
        f"verify {m['verify_us']:.2f} us; hot: {m['hot_us']:.2f} us/call, "
        f"verify {m['hot_verify_us']:.2f} us")
    gbs = b.kv_bytes / (m["us"] * 1e-6) / 1e9
    achieved = b.kv_bytes / (m["verify_us"] * 1e-6) / 1e9
    outputs = {w.name: (w, m.pop("out"))}
    combines = b.time_combines()
    log(f"[bench] combine {combines['combine_us']:.2f} us, with LSE {combines['combine_lse_us']:.2f} us")
    plan = b.plan
    del b
    torch.cuda.empty_cache()

    sweep = []
    if not args.no_sweep:
        steps = max(20, args.steps // 2)
        for name in ["c1", "c2_16k", "c2_32k", "c2_64k", "c2_128k"]:
            log(f"[bench] sweep {name}")
            ws = wl.cached(name)
            bs = DenseBench(ws, copies_for(ws.kv_bytes()), args.kernel, 0)
            ms = measure(bs, steps, args.warmup)
            outputs[ws.name] = (ws, ms.pop("out"))
            sweep.append(sweep_entry(ws.name, bs.kv_bytes, bs.plan, ms, ctx=ws.max_tokens))
            del bs
            torch.cuda.empty_cache()
        log("[bench] sweep c4 (QSA)")
        wq = wl.cached("c4")
        bq = QsaBench(wq, copies_for(wq.kv_bytes()), args.kernel)
        mq = measure(bq, steps, args.warmup)
        outputs[wq.name] = (wq, mq.pop("out"))
        sweep.append(sweep_entry(wq.name, bq.kv_bytes, bq.plan, mq,
                                 units=wq.batch * wq.num_kv_heads))
        del bq
        torch.cuda.empty_cache()
        log("[bench] sweep c4tok (QSA over token ids)")
        wt = wl.cached("c4tok")
        bt = QsaTokensBench(wt, copies_for(wt.kv_bytes()), args.kernel)
        mt = measure(bt, steps, args.warmup)
        outputs[wt.name] = (wt, mt.pop("out"))
        sweep.append(sweep_entry(wt.name, bt.kv_bytes, bt.plan, mt,
                                 units=wt.batch * wt.num_kv_heads))
        del bt
        torch.cuda.empty_cache()
        log("[bench] sweep batch (independent requests)")
        wb = wl.cached("batch")
        bb = BatchBench(wb, copies_for(wb.kv_bytes()), args.kernel)
        mb = measure(bb, steps, args.warmup)
        outputs[wb.name] = (wb, mb.pop("out"))
        sweep.append(sweep_entry(wb.name, bb.kv_bytes, bb.plan, mb,
                                 units=wb.batch * wb.num_kv_heads))
        del bb
        torch.cuda.empty_cache()
        sweep.append(sweep_entry(w.name, w.kv_bytes(), plan, m, ctx=w.max_tokens))
        for e in sweep:
            e["traffic"] = traffic_from_profile(src_hash, e["workload"])

    cache_write = None
    if not args.no_sweep:
        log("[bench] E4M3 cache write")
        cache_write = [time_cache_write(torch, pa, t) for t in (8, 4096, 65536)]
        torch.cuda.empty_cache()

    log("[bench] streaming-read ceiling")
    ceiling = read_ceiling(torch, pa)
    same_size = read_ceiling_at(torch, pa, w.kv_bytes())
    log(f"[bench] read probe over {w.kv_bytes()} B, cold: {same_size['us']:.2f} us, "
        f"{same_size['gbs']:.0f} GB/s")

    cpu, accuracy = None, None
    if not args.no_cpu_baseline:
        log("[bench] cpu baseline (oracle), and the oracle's outputs for the accuracy figures")
        cpu, accuracy = cpu_baseline(w, outputs)

    kernel_name = {0: "auto", 1: "simple", 2: "mfma"}[plan.kernel]
    traffic = traffic_from_profile(src_hash, w.name)
    line = {
        "metric": METRIC,
        "value": round(gbs, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(m["us"] * 1e-3, 6),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f16" if kernel_name != "simple" else "f32",
        "data": "synthetic",
        "config": {"workload": w.name, "q_rows": w.q_rows, "num_heads": w.num_heads,
                   "num_kv_heads": w.num_kv_heads, "head_dim": w.head_dim,
                   "ctx": w.max_tokens, "page_size": w.page_size, "kv_bytes": w.kv_bytes(),
                   "splits": plan.num_splits, "tokens_per_split": plan.tokens_per_split,
                   "rows_per_workgroup": plan.rows_per_workgroup, "kernel": kernel_name, "cache": f"cold: {n_copies} rotating pool copies",
                   "us_per_call": round(m["us"], 3), "timing": "HIP graph of 10 verify + combine calls, replayed",
                   "pct_hbm_peak": round(100 * gbs / HBM_PEAK_GBS, 2)},
        "hot": {"us_per_call": round(m["hot_us"], 3),
                "value": round(w.kv_bytes() / (m["hot_us"] * 1e-6) / 1e9, 2),
                "verify_us": round(m["hot_verify_us"], 3), "us_per_call_pcts": m["hot_pcts"]},
        "us_per_call_pcts": m["pcts"],
        "eager_us_per_call": round(m["eager_us"], 3),
        "roofline": {"bound": "hbm", "achieved": round(achieved, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(achieved / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": "verify", "verify_us": round(m["verify_us"], 3),
                     "verify_us_median": round(m["verify_med_us"], 3),
                     "read_ceiling": ceiling,
                     "frac_of_read_ceiling": round(achieved / ceiling, 4) if ceiling else None,
                     "read_probe_same_bytes": same_size,
                     "frac_of_read_probe_same_bytes": round(same_size["us"] / m["verify_us"], 4)},
        "combine": combines,
        "cache_write": cache_write,
        "cpu_baseline": cpu,
        "accuracy": accuracy,
        "sweep": sweep,
        "source_hash": src_hash,
        "build_id": pa.build_id(),
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
