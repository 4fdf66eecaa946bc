"""Benchmark of the sliding-window attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W]
                    [--workload all|c1|c2|c2w|c3|c3w|c4|c5|evict|alloc|unified] [--window W]

Default (all): one JSON line whose headline is the largest single-GPU
configuration, the long-context mixed-layer decode step (B = 32, T = 32K, 48
layers: 39 SWA layers with W = 128 and 8 kv heads, 9 full-attention layers with
4 kv heads, 64 q heads, head_dim 128, bf16, page 64, SWA pool at ratio 0.1):
    swa_decode_step: the window table once (req_to_token -> full -> SWA
    slots), then the 48 layers in order through the layers mapping (SWA
    layers: windowed decode over the shared table; full layers: split-K decode
    over req_to_token + merge).
The same line carries the other configurations as sub-results, each with its
own roofline and CPU baseline:
    c2   batched SWA decode, B = 64, T ~ U[1K, 8K], W = 128, 64 q / 8 kv, bf16,
         page 16, with the new token's store fused (32 layers per step)
    c5   fp8-KV SWA decode, B = 256, lognormal T (median 16K), e4m3 K/V, page 64,
         translate + store + decode (16 layers per step)
    c2w  the c2 batch with W = 1023 and 4095 (long windows, split over their keys;
         8 layers per step)
    c3   chunked-prefill extend, B = 4, prefix 8K + chunk 2K, W = 128, page 64,
         store + extend (4 layers per step): TFLOP/s, fraction of MFMA peak and of
         the attainable roofline
    c3w  the c3 shape with W = 512, 1024, 4096 (compute-bound windows)
    c1   one f32 request, T = 512, W = 128 (latency)
Before the workloads, three probes of the library (include/swa_probe.h) measure
the practical ceilings, a streaming read, a copy and a bf16 MFMA loop, and every
roofline is also stated as a fraction of them (`probes`, `frac_of_probe`).
Every step is captured once as a HIP graph and replayed; inputs are resident in
HBM before the timed region.  `value` is algorithmic HBM bytes of the whole step
per second.  Each `roofline` is its dominant kernel, timed live with HIP events
around back-to-back graph replays on the replay stream.  Each `cpu_baseline` is
the CPU oracle as it stands, run on a process pool of one worker per host core
(at most 16, BLAS at one thread each) over a bounded sample of the same work,
before the GPU is first touched.

Single workloads (--workload NAME) print their own line in the same format;
evict, alloc and unified are the next-row kernels (eviction, paired allocation,
unified pool layout).
"""

from __future__ import annotations

import argparse
import hashlib
import itertools
import json
import math
import multiprocessing
import os
import re
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
SIMDS = 1024                 # 256 CUs x 4 SIMDs
METRIC = "SWA decode HBM GB/s & tokens/s; windowed prefill TFLOP/s (% of MI355X peak)"
SWEEP_WINDOWS = (512, 1024, 4096)   # prefill window sweep on the C3 shape
DECODE_WINDOWS = (1023, 4095)       # long-window decode on the C2 batch


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def code_text(src: str) -> str:
    """Source text without comments and blank space, so that a sha of it changes
    with the code only (the kernels hold no string literals with comment marks)."""
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    return " ".join(src.split())


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sliding_window_attention_swa_amd", "csrc", n), encoding="utf-8") as f:
            h.update(code_text(f.read()).encode())
    return h.hexdigest()[:16]


DECODE_SRC = ["decode_kernels.hip", "common.hpp", "api.cpp"]
EXTEND_SRC = ["extend_kernels.hip", "common.hpp", "api.cpp"]


def profile_record(name: str, kernel_files):
    """A committed rocprofv3 counter summary (profiles/<name>_pmc.json), or None
    when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != source_sha(*kernel_files):
        return None
    return d


def traffic_from_profile(name: str, kernel_files):
    d = profile_record(name, kernel_files)
    return None if d is None else d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, on a fork pool of one process per host
# core (at most 16: the host share of one GPU), BLAS limited to one thread per
# process, over a bounded sample of the benchmarked work.  It runs before the GPU
# is first used; the workers inherit the host inputs in _HOST.
# ---------------------------------------------------------------------------

_HOST = {}
CPU_BUDGET_S = 20.0   # CPU seconds of oracle work per measured item (wall = budget / workers)


def cpu_workers() -> int:
    return max(1, min(len(os.sched_getaffinity(0)), 16))


def _worker_init():
    from threadpoolctl import threadpool_limits
    threadpool_limits(1)


def _cpu_task(task):
    """One task of oracle work on the host inputs in _HOST."""
    from oracle import swa_oracle as O
    kind, name = task[0], task[1]
    d = _HOST[name]
    if kind == "decode":          # one request of one layer, every q head
        wl, b = d, task[2]
        O.decode(wl.q, wl.q_dtype, wl.pool_k, wl.pool_v, wl.kv_dtype, wl.req_to_token, wl.req_pool_idx,
                 wl.seq_lens, wl.full_to_swa, wl.window, wl.sinks, only=[(b, h) for h in range(wl.q_heads)])
    elif kind == "store":         # translate + store of the new rows + window table, whole batch, one layer
        wl = d
        loc = wl.new_full_loc if wl.full_to_swa is None else O.translate_loc(wl.new_full_loc, wl.full_to_swa)
        O.kv_store(wl.pool_k, wl.pool_v, loc, wl.new_k, wl.new_v, wl.new_dtype, wl.kv_dtype)
        O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window,
                       prefix_lens=wl.prefix_lens)
    elif kind == "extend":        # query rows r0 .. r1-1 of one layer, every q head
        wl, r0, r1 = d, task[2], task[3]
        O.extend(wl.q, "bf16", wl.qo_indptr, wl.prefix_lens, wl.pool_k, wl.pool_v, "bf16", wl.req_to_token,
                 wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window, wl.sinks,
                 only=[(r, h) for r in range(r0, r1) for h in range(wl.q_heads)])
    elif kind == "mixed":         # one request of one full or SWA layer of the mixed step, every q head
        part, b = task[2], task[3]
        x = d[part]
        O.decode(x["q"], "bf16", x["k"], x["v"], "bf16", d["r2t"], d["rows"], d["lens"], x["map"], x["window"],
                 None, only=[(b, h) for h in range(d["q_heads"])])
    else:
        raise ValueError(kind)
    return 1


def pool_time(pool, nw, tasks, unit_tasks):
    """Wall time of whole units of `tasks` (each unit is `unit_tasks` tasks, in
    order) on the pool, sized to about CPU_BUDGET_S of oracle work: the number
    of units grows from one (after one untimed unit) until a run lasts about
    CPU_BUDGET_S / workers seconds; the last run is the measurement.  Returns
    (units, seconds)."""
    target = CPU_BUDGET_S / nw
    pool.map(_cpu_task, tasks[:unit_tasks], chunksize=1)   # warm-up: first touch of the inputs in every worker
    units = 1
    while True:
        work = list(itertools.islice(itertools.cycle(tasks[:unit_tasks]), units * unit_tasks))
        chunk = max(1, min(8, len(work) // (4 * nw)))
        t0 = time.perf_counter()
        pool.map(_cpu_task, work, chunksize=chunk)
        secs = time.perf_counter() - t0
        if secs >= 0.5 * target or units >= 1 << 20:
            return units, secs
        units = max(2 * units, int(units * target / max(secs, 1e-3)))


def cpu_decode_layer(pool, nw, name, wl):
    """Layers of decode work per second: the batch's store and window table,
    then every request's decode."""
    tasks = ([("store", name)] if wl.new_full_loc is not None else []) + [("decode", name, b)
                                                                           for b in range(wl.batch)]
    return pool_time(pool, nw, tasks, len(tasks))


def cpu_extend_layer(pool, nw, name, wl, rows_per_task):
    """Extend query rows per second (every q head): a unit is one task of
    `rows_per_task` consecutive rows per worker, the tasks spread over the
    chunk."""
    total = wl.q.shape[0]
    starts = np.linspace(0, total - rows_per_task, nw).astype(int)
    tasks = [("extend", name, int(r), int(r) + rows_per_task) for r in starts]
    units, secs = pool_time(pool, nw, tasks, len(tasks))
    return units * len(tasks) * rows_per_task, secs


def mixed_host_data(st, full_sample=4, seed=97):
    """Host inputs of the mixed step's oracle sample: one full layer holding the
    K/V rows of `full_sample` requests, one SWA layer holding every request's
    window (values drawn here; the oracle reads them as it reads any pool)."""
    from sliding_window_attention_swa_amd import workloads as W
    from oracle import swa_oracle as O
    rng = np.random.default_rng(seed)
    B, Hq, D, T = st.batch, st.q_heads, st.head_dim, int(st.seq_lens[0])
    r2t, rows = st.req_to_token, st.req_pool_idx
    sample = list(range(0, B, B // full_sample))[:full_sample]
    used_f = np.unique(np.concatenate([r2t[rows[b], :T] for b in sample]).astype(np.int64))
    used_s = np.unique(np.concatenate([O.translate_loc(r2t[rows[b], T - 129:T], st.full_to_swa) for b in range(B)]))
    draw = lambda n, h: W.to_store(rng.standard_normal((n, h, D), dtype=np.float32), "bf16")  # noqa: E731
    full = dict(q=draw(B, Hq), map=None, window=-1,
                k=W.SparsePool(st.n_full + st.page_size, 4, D, "bf16", used_f, draw(used_f.size, 4)),
                v=W.SparsePool(st.n_full + st.page_size, 4, D, "bf16", used_f, draw(used_f.size, 4)))
    swl = dict(q=draw(B, Hq), map=st.full_to_swa, window=128,
               k=W.SparsePool(st.n_swa + st.page_size, 8, D, "bf16", used_s, draw(used_s.size, 8)),
               v=W.SparsePool(st.n_swa + st.page_size, 8, D, "bf16", used_s, draw(used_s.size, 8)))
    return dict(full=full, swa=swl, r2t=r2t, rows=rows, lens=st.seq_lens, q_heads=Hq, sample=sample, batch=B)


def cpu_mixed_step(pool, nw, d):
    """The 48-layer step's oracle time: a full layer over the sampled requests
    and an SWA layer over every request, timed on the pool; the step is 9 full
    plus 39 SWA layers over all 32 requests."""
    B, sample, full_sample = d["batch"], d["sample"], len(d["sample"])
    n_full, t_full = pool_time(pool, nw, [("mixed", "c4", "full", b) for b in sample], len(sample))
    n_swa, t_swa = pool_time(pool, nw, [("mixed", "c4", "swa", b) for b in range(B)], B)
    per_full = t_full / (n_full * len(sample))        # seconds per (request, full layer) on the pool
    per_swa = t_swa / (n_swa * B)
    step_s = B * (9 * per_full + 39 * per_swa)
    return step_s, (f"one full layer (32K keys, 4 kv heads) on {full_sample} of {B} requests, {n_full} times, "
                    f"and one SWA layer on all {B} requests, {n_swa} times, every q head; step time = "
                    f"{B} requests x (9 x {per_full * 1e3:.2f} ms + 39 x {per_swa * 1e3:.3f} ms per request and layer)")


def cpu_baseline_entry(value, unit, nw, sample):
    return dict(value=value, unit=unit, cores=nw, kind="oracle", sample=sample)


def run_cpu_baselines(names, hosts):
    """The oracle timed for each named workload (host inputs in `hosts`), before
    any GPU use.  Returns {name: cpu_baseline dict}."""
    nw = cpu_workers()
    # the workers see what _HOST holds when the pool forks
    for name in names:
        _HOST[name] = mixed_host_data(hosts[name]["st"]) if name == "c4" else hosts[name]["wl"]
    ctx = multiprocessing.get_context("fork")
    out = {}
    with ctx.Pool(nw, initializer=_worker_init) as pool:
        pool.map(abs, range(nw), chunksize=1)  # every worker started before the timing
        for name in names:
            t0 = time.perf_counter()
            h = hosts[name]
            if name == "c4":
                step_s, sample = cpu_mixed_step(pool, nw, _HOST["c4"])
                out[name] = cpu_baseline_entry(round(h["step_bytes"] / step_s / 1e9, 6), "GB/s", nw, sample)
                out[name]["tokens_per_s"] = round(h["st"].batch / step_s, 4)
            elif name in ("c1", "c2", "c5") or name.startswith("c2w_"):
                wl = h["wl"]
                units, secs = cpu_decode_layer(pool, nw, name, wl)
                out[name] = cpu_baseline_entry(round(units * h["layer_bytes"] / secs / 1e9, 6), "GB/s", nw,
                                               f"{units} layers of {wl.batch} requests (translate + store + window "
                                               f"table, then every request's decode, every q head) in {secs:.2f} s")
                out[name]["tokens_per_s"] = round(units * wl.batch / h["layers"] / secs, 4)
            else:  # c3, c3w_<W>
                wl = h["wl"]
                rows, secs = cpu_extend_layer(pool, nw, name, wl, h["rows_per_task"])
                flops = rows * h["flops_per_row"]
                out[name] = cpu_baseline_entry(round(flops / secs / 1e12, 9), "TFLOP/s", nw,
                                               f"{rows} query rows x {wl.q_heads} q heads of the extend "
                                               f"(W = {wl.window}) in {secs:.2f} s")
            log(f"[cpu] {name}: {out[name]['value']} {out[name]['unit']} on {nw} processes "
                f"({time.perf_counter() - t0:.1f} s)")
    _HOST.clear()
    return out


# ---------------------------------------------------------------------------
# device setup helpers (torch for memory only)
# ---------------------------------------------------------------------------


def randn_store(torch, shape, gen, dtype):
    x = torch.randn(shape, generator=gen, device="cuda")
    if dtype == "bf16":
        return x.to(torch.bfloat16)
    if dtype == "e4m3":
        return x.to(torch.float8_e4m3fn).view(torch.uint8)
    return x


def nan_pool(torch, rows, H, D, dtype):
    if dtype == "bf16":
        t = torch.empty((rows, H, D), dtype=torch.bfloat16, device="cuda")
        t.view(torch.int16).fill_(0x7FC0)
    elif dtype == "e4m3":
        t = torch.full((rows, H, D), 0x7F, dtype=torch.uint8, device="cuda")
    else:
        t = torch.full((rows, H, D), float("nan"), dtype=torch.float32, device="cuda")
    return t


def graph_of(torch, fn):
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        fn()  # eager run on the side stream before capture
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


def time_replays(torch, g, n):
    start, end = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    start.record()
    for _ in range(n):
        g.replay()
    end.record()
    torch.cuda.synchronize()
    return start.elapsed_time(end) / n  # ms per replay


def replay_percentiles(torch, g, n, per_replay):
    """p10 / p50 / p90 of one replay's duration (ms), each replay bracketed by
    its own pair of events on the stream the graph is replayed on, divided by
    the `per_replay` launches it holds."""
    ev = [torch.cuda.Event(enable_timing=True) for _ in range(n + 1)]
    torch.cuda.synchronize()
    ev[0].record()
    for i in range(n):
        g.replay()
        ev[i + 1].record()
    torch.cuda.synchronize()
    d = np.array([ev[i].elapsed_time(ev[i + 1]) for i in range(n)]) / per_replay
    return {k: round(float(np.percentile(d, q)) * 1e3, 3) for k, q in (("p10_us", 10), ("p50_us", 50), ("p90_us", 90))}


def timed_step(torch, fn, steps, warmup):
    g = graph_of(torch, fn)
    for _ in range(warmup):
        g.replay()
    return time_replays(torch, g, steps)


def timed_dominant(torch, fn, reps, per_replay):
    g = graph_of(torch, fn)
    g.replay()
    ms = time_replays(torch, g, reps) / per_replay
    return ms, replay_percentiles(torch, g, reps, per_replay)


# ---------------------------------------------------------------------------
# decode workloads (c1, c2, c5): one batch replicated over `layers` SWA layers
# ---------------------------------------------------------------------------


def decode_host(name):
    from sliding_window_attention_swa_amd import workloads as W
    if name == "c2":
        return W.c2_decode_bf16(), 32, "batched SWA decode B=64, T~U[1K,8K], W=128, 64q/8kv, D=128, bf16, page 16"
    if name.startswith("c2w_"):
        w = int(name.split("_")[1])
        return (W.c2_decode_bf16(window=w), 8,
                f"long-window SWA decode: the B=64 batch of T~U[1K,8K] with W={w}, 64q/8kv, D=128, bf16, page 16, "
                "split over the window's keys")
    if name == "c5":
        return (W.c5_decode_fp8(), 16,
                "fp8 KV decode B=256, T~lognormal(16K), W=128, 64q/8kv, D=128, e4m3 K/V, bf16 q, page 64")
    return W.c1_decode_f32(), 8, "single SWA decode T=512, W=128, 8q/8kv, D=128, f32, page 1"


def decode_bytes(wl, out_dtype):
    """Algorithmic bytes of one layer's decode (window only: K/V rows, Q, O,
    window table) and of its store (the new rows written; read as the window's
    last row when fused)."""
    B, Hq, Hkv, D = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    n_keys = np.minimum(wl.seq_lens.astype(np.int64), wl.window + 1)
    kv_b = {"bf16": 2, "e4m3": 1, "f32": 4}[wl.kv_dtype]
    q_b = {"bf16": 2, "f32": 4}[wl.q_dtype]
    o_b = 2 if out_dtype == "bf16" else 4
    dec = int(n_keys.sum() * Hkv * D * kv_b * 2 + B * Hq * D * (q_b + o_b) + n_keys.sum() * 4 + (B + 1) * 4)
    new_b = 2 if wl.kv_dtype != "f32" else 4
    fused = wl.new_full_loc is not None and wl.kv_dtype == "bf16" and 0 <= wl.window <= 255
    if wl.new_full_loc is None:
        store = 0
    elif fused:
        store = B * Hkv * D * kv_b * 2 + B * 8
    else:
        store = B * Hkv * D * 2 * (new_b + kv_b) + B * 8
    translate = (B * 8 * 3 if wl.new_full_loc is not None else 0) + int(n_keys.sum()) * (4 + 8 + 4) + B * 12
    return dec, store, translate, fused, int(n_keys.sum()) * Hq * D * 4


class DecodeBench:
    """A decode batch of one workload replicated over `layers` SWA layers, each
    with its own pools (so the 256 MB Infinity Cache cannot serve repeats)."""

    def __init__(self, torch, swa, wl, layers, out_dtype="bf16", seed=7):
        self.torch, self.swa, self.wl, self.L = torch, swa, wl, layers
        B, Hq, Hkv, D = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
        self.r2t = torch.from_numpy(wl.req_to_token).cuda()
        self.rows = torch.from_numpy(wl.req_pool_idx).cuda()
        self.lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
        self.map = torch.from_numpy(wl.full_to_swa).cuda()
        self.index = swa.IndexTables(self.r2t, self.rows, self.lens, self.map, wl.page_size)
        self.has_store = wl.new_full_loc is not None
        if self.has_store:
            self.full_loc = torch.from_numpy(wl.new_full_loc).cuda()
            self.swa_loc = torch.empty_like(self.full_loc)
        self.cap = B * (wl.window + 1)
        self.table = torch.empty(self.cap, dtype=torch.int32, device="cuda")
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        used = torch.from_numpy(wl.pool_k.used_rows).cuda()
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.layers = []
        for _ in range(layers):
            k = nan_pool(torch, wl.pool_rows, Hkv, D, wl.kv_dtype)
            v = nan_pool(torch, wl.pool_rows, Hkv, D, wl.kv_dtype)
            k[used] = randn_store(torch, (used.numel(), Hkv, D), g, wl.kv_dtype)
            v[used] = randn_store(torch, (used.numel(), Hkv, D), g, wl.kv_dtype)
            new_dt = "bf16" if wl.kv_dtype != "f32" else "f32"
            self.layers.append(dict(
                kv=swa.KvLayer(k, v), q=randn_store(torch, (B, Hq, D), g, wl.q_dtype),
                new_k=randn_store(torch, (B, Hkv, D), g, new_dt), new_v=randn_store(torch, (B, Hkv, D), g, new_dt),
                out=torch.empty((B, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                                device="cuda")))
        self.sinks = torch.from_numpy(wl.sinks).cuda() if wl.sinks is not None else None
        self.decode_bytes, self.store_bytes, self.translate_bytes, self.fused, self.flops = decode_bytes(wl, out_dtype)
        # windows past the one-split kernels: the library's plan (split over the window's keys)
        self.splits, ws = swa.swa_decode_plan(B, Hq, Hkv, D, wl.window, int(wl.seq_lens.max()))
        self.ws = torch.empty(max(ws // 4, 1), dtype=torch.float32, device="cuda") if ws > 0 else None
        self.step_bytes = self.translate_bytes + layers * (self.store_bytes + self.decode_bytes)

    def step(self):
        swa, wl = self.swa, self.wl
        if self.has_store:
            swa.swa_translate_loc(self.full_loc, self.map, self.swa_loc)
        swa.swa_translate_window(self.index, wl.window, self.table, self.indptr)
        for ly in self.layers:
            if self.has_store and not self.fused:
                swa.swa_kv_store(ly["kv"], self.swa_loc, ly["new_k"], ly["new_v"])
            self.decode_call(ly)

    def decode_call(self, ly):
        swa, wl = self.swa, self.wl
        if self.fused:
            swa.swa_decode_store(ly["q"], ly["kv"], self.index, wl.window, ly["out"], self.swa_loc, ly["new_k"],
                                 ly["new_v"], sinks=self.sinks, slot_table=self.table, table_indptr=self.indptr)
        else:
            swa.swa_decode(ly["q"], ly["kv"], self.index, wl.window, ly["out"], sinks=self.sinks,
                           slot_table=self.table, table_indptr=self.indptr, num_splits=self.splits,
                           workspace=self.ws)

    def dominant(self):
        """Back-to-back decode launches only (one per layer; with the store fused
        in when the step fuses it)."""
        for ly in self.layers:
            self.decode_call(ly)


def run_decode_gpu(args, torch, swa, name, wl, layers, desc, cpu):
    out_dtype = "f32" if wl.q_dtype == "f32" else "bf16"
    log(f"[bench] {name}: building {layers} layers")
    bench = DecodeBench(torch, swa, wl, layers, out_dtype)
    ms = timed_step(torch, bench.step, args.steps, args.warmup)
    reps = max(10, args.steps // 2)
    ms_dec, pct = timed_dominant(torch, bench.dominant, reps, layers)
    log(f"[bench] {name}: step {ms:.4f} ms, decode {ms_dec * 1e3:.2f} us per launch")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    dom_bytes = bench.decode_bytes + (bench.store_bytes if bench.fused else 0)
    achieved = dom_bytes / (ms_dec * 1e-3) / 1e9
    res = dict(
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 5), dtype={"c5": "bf16 q / e4m3 kv",
                                                                            "c1": "f32"}.get(name, "bf16"),
        config={"workload": desc, "global_batch": int(wl.batch), "layers_per_step": layers, "window": wl.window,
                "max_seq_len": int(wl.seq_lens.max()), "num_splits": bench.splits},
        tokens_per_s=round(wl.batch / (ms * 1e-3), 1),
        layer_tokens_per_s=round(wl.batch * layers / (ms * 1e-3), 1),
        roofline=dict(kernel="swa_decode_store (store fused)" if bench.fused else
                      "swa_decode (split over the window's keys: stream + merge)" if wl.window > 255 else "swa_decode",
                      bound="hbm",
                      achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile(f"swa_decode_{name}", DECODE_SRC),
                      bytes_per_launch=dom_bytes, us_per_launch=round(ms_dec * 1e3, 3), **pct),
    )
    if name == "c1":
        res["roofline"]["note"] = "latency configuration: 1 MB per launch, far below what fills the chip"
    if cpu is not None:
        res["cpu_baseline"] = cpu
    del bench
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# extend workloads (c3 and the window sweep)
# ---------------------------------------------------------------------------


def extend_counts(wl):
    """Band-only FLOPs and algorithmic bytes of one extend launch, and of the
    store of the chunk."""
    B, Hq, Hkv, D = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
    total_q = wl.q.shape[0]
    lo = np.maximum(wl.prefix_lens.astype(np.int64) - wl.window, 0)
    n_keys = wl.seq_lens.astype(np.int64) - lo
    pairs = 0
    for b in range(B):
        i = np.arange(int(wl.prefix_lens[b]), int(wl.seq_lens[b]))
        pairs += int(np.sum(i - np.maximum(i - wl.window, 0) + 1))
    flops = pairs * Hq * D * 4
    ext_bytes = int(total_q * Hq * D * 2 * 2 + n_keys.sum() * Hkv * D * 2 * 2 + n_keys.sum() * 4
                    + (B + 1) * 4 * 2 + B * 4 * 2)
    store_bytes = total_q * Hkv * D * 2 * 2 * 2 + total_q * 8
    return flops, ext_bytes, store_bytes, int(n_keys.sum())


class ExtendBench:
    """An extend batch replicated over `layers` SWA layers."""

    def __init__(self, torch, swa, wl, layers, seed=11):
        self.torch, self.swa, self.wl = torch, swa, wl
        B, Hq, Hkv, D = wl.batch, wl.q_heads, wl.kv_heads, wl.head_dim
        self.r2t = torch.from_numpy(wl.req_to_token).cuda()
        self.rows = torch.from_numpy(wl.req_pool_idx).cuda()
        self.lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).cuda()
        self.map = torch.from_numpy(wl.full_to_swa).cuda()
        self.prefix = torch.from_numpy(wl.prefix_lens).cuda()
        self.qo = torch.from_numpy(wl.qo_indptr).cuda()
        self.index = swa.IndexTables(self.r2t, self.rows, self.lens, self.map, wl.page_size)
        self.full_loc = torch.from_numpy(wl.new_full_loc).cuda()
        self.swa_loc = torch.empty_like(self.full_loc)
        self.extend_flops, self.extend_bytes, self.store_bytes, self.cap = extend_counts(wl)
        self.table = torch.empty(self.cap, dtype=torch.int32, device="cuda")
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        used = torch.from_numpy(wl.pool_k.used_rows).cuda()
        total_q = wl.q.shape[0]
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        self.layers = []
        for _ in range(layers):
            k = nan_pool(torch, wl.pool_rows, Hkv, D, "bf16")
            v = nan_pool(torch, wl.pool_rows, Hkv, D, "bf16")
            k[used] = randn_store(torch, (used.numel(), Hkv, D), g, "bf16")
            v[used] = randn_store(torch, (used.numel(), Hkv, D), g, "bf16")
            self.layers.append(dict(kv=swa.KvLayer(k, v), q=randn_store(torch, (total_q, Hq, D), g, "bf16"),
                                    new_k=randn_store(torch, (total_q, Hkv, D), g, "bf16"),
                                    new_v=randn_store(torch, (total_q, Hkv, D), g, "bf16"),
                                    out=torch.empty((total_q, Hq, D), dtype=torch.bfloat16, device="cuda")))
        self.sinks = torch.from_numpy(wl.sinks).cuda()
        self.step_bytes = total_q * 8 * 3 + self.cap * 16 + layers * (self.store_bytes + self.extend_bytes)
        self.step_flops = layers * self.extend_flops

    def step(self):
        swa, wl = self.swa, self.wl
        swa.swa_translate_loc(self.full_loc, self.map, self.swa_loc)
        swa.swa_translate_window(self.index, wl.window, self.table, self.indptr, prefix_lens=self.prefix)
        for ly in self.layers:
            swa.swa_kv_store(ly["kv"], self.swa_loc, ly["new_k"], ly["new_v"])
            self.extend_call(ly)

    def extend_call(self, ly):
        self.swa.swa_extend(ly["q"], self.qo, self.prefix, ly["kv"], self.index, self.wl.window, ly["out"],
                            sinks=self.sinks, slot_table=self.table, table_indptr=self.indptr)

    def dominant(self):
        for ly in self.layers:
            self.extend_call(ly)


def extend_host(window=128):
    from sliding_window_attention_swa_amd import workloads as W
    return W.c3_extend_bf16(window=window)


def run_extend_gpu(args, torch, swa, name, wl, cpu, layers=4):
    log(f"[bench] {name}: building {layers} layers (W = {wl.window})")
    bench = ExtendBench(torch, swa, wl, layers)
    ms = timed_step(torch, bench.step, args.steps, args.warmup)
    reps = max(5, args.steps)
    ms_ext, pct = timed_dominant(torch, bench.dominant, reps, layers)
    log(f"[bench] {name}: step {ms:.4f} ms, extend {ms_ext * 1e3:.2f} us")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    achieved_gbs = bench.extend_bytes / (ms_ext * 1e-3) / 1e9
    tflops = bench.extend_flops / (ms_ext * 1e-3) / 1e12
    intensity = bench.extend_flops / bench.extend_bytes
    attainable = min(BF16_PEAK_TFLOPS, intensity * HBM_PEAK_GBS / 1e3)
    bound = "hbm" if intensity * HBM_PEAK_GBS / 1e3 < BF16_PEAK_TFLOPS else "mfma"
    prof = profile_record(f"swa_extend_{name}", EXTEND_SRC)
    roof = dict(kernel="swa_extend", bound=bound, flops_per_launch=bench.extend_flops,
                bytes_per_launch=bench.extend_bytes, us_per_launch=round(ms_ext * 1e3, 3), **pct,
                tflops=round(tflops, 2), frac_of_mfma_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
                attainable_tflops=round(attainable, 1), frac_of_attainable=round(tflops / attainable, 4),
                achieved_gbs=round(achieved_gbs, 1), frac_of_hbm_peak=round(achieved_gbs / HBM_PEAK_GBS, 4),
                traffic=None if prof is None else prof.get("hbm_bytes_per_launch"),
                mfma_busy_counter=None if prof is None else prof.get("mfma_busy_frac"))
    if bound == "hbm":
        roof.update(achieved=round(achieved_gbs, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                    frac=round(achieved_gbs / HBM_PEAK_GBS, 4))
    else:
        roof.update(achieved=round(tflops, 2), peak=BF16_PEAK_TFLOPS, unit="TFLOP/s",
                    frac=round(tflops / BF16_PEAK_TFLOPS, 4))
    res = dict(
        value=round(bench.step_flops / (ms * 1e-3) / 1e12, 2), unit="TFLOP/s", step_gbs=round(value, 1),
        ms_per_step=round(ms, 5), dtype="bf16",
        config={"workload": f"chunked-prefill extend B={wl.batch}, prefix 8K + chunk 2K, W={wl.window}, 64q/8kv, "
                            f"D=128, bf16, page 64 (store + extend per layer)", "global_batch": int(wl.batch),
                "new_tokens": int(wl.q.shape[0]), "layers_per_step": layers, "window": wl.window},
        tokens_per_s=round(wl.q.shape[0] * layers / (ms * 1e-3), 1),
        roofline=roof,
    )
    if cpu is not None:
        res["cpu_baseline"] = cpu
    del bench
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# c4: 48-layer mixed decode step (39 SWA + 9 full layers) through swa_decode_step
# ---------------------------------------------------------------------------


def mixed_bytes(st):
    B, Hq, D, T, W1 = st.batch, st.q_heads, st.head_dim, int(st.seq_len), 129
    full = B * T * 4 * D * 2 * 2 + B * Hq * D * 4 + B * T * 4
    swl = B * W1 * 8 * D * 2 * 2 + B * Hq * D * 4 + B * W1 * 4
    return full, swl, 9 * full + 39 * swl + B * W1 * 16


class MixedBench:
    def __init__(self, torch, swa, st):
        from sliding_window_attention_swa_amd import workloads as W
        self.torch, self.swa, self.st = torch, swa, st
        B, Hq, D = st.batch, st.q_heads, st.head_dim
        self.index = swa.IndexTables(torch.from_numpy(st.req_to_token).cuda(),
                                     torch.from_numpy(st.req_pool_idx).cuda(), torch.from_numpy(st.seq_lens).cuda(),
                                     torch.from_numpy(st.full_to_swa).cuda(), st.page_size)
        self.table = torch.empty(B * 129, dtype=torch.int32, device="cuda")
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        full_ids = [ly["id"] for ly in st.layers if ly["kind"] == "full"]
        swa_ids = [ly["id"] for ly in st.layers if ly["kind"] == "swa"]
        self.mapping = [(full_ids.index(ly["id"]), 0) if ly["kind"] == "full" else (swa_ids.index(ly["id"]), 1)
                        for ly in st.layers]
        tensors = [W.c4_layer_tensors(st, ly) for ly in st.layers]
        self.full_layers = [swa.KvLayer(tensors[i][1], tensors[i][2]) for i in full_ids]
        self.swa_layers = [swa.KvLayer(tensors[i][1], tensors[i][2]) for i in swa_ids]
        self.q = [t[0] for t in tensors]
        self.out = [torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda") for _ in st.layers]
        self.dstep = swa.DecodeStep(self.mapping, self.full_layers, self.swa_layers, 128, self.q, self.out)
        self.ws = torch.empty(max(self.dstep.workspace_bytes(self.index, st.seq_len) // 4, 1), dtype=torch.float32,
                              device="cuda")
        self.splits, _ = swa.swa_decode_plan(B, Hq, 4, D, -1, st.seq_len)
        self.full_ids = full_ids
        self.full_bytes, self.swa_bytes, self.step_bytes = mixed_bytes(st)

    def step(self):
        self.swa.swa_decode_step(self.dstep, self.index, self.st.seq_len, self.table, self.indptr, self.ws)

    def dominant(self):
        """The full layers' decodes only (split-K + merge), as the step issues them."""
        for i, lid in enumerate(self.full_ids):
            self.swa.swa_decode(self.q[lid], self.full_layers[i], self.index, -1, self.out[lid],
                                num_splits=self.splits, workspace=self.ws, use_map=False)


def run_mixed_gpu(args, torch, swa, st, cpu):
    log("[bench] c4: building 48 layers")
    bench = MixedBench(torch, swa, st)
    ms = timed_step(torch, bench.step, args.steps, args.warmup)
    reps = max(3, args.steps // 2)
    ms_full, pct = timed_dominant(torch, bench.dominant, reps, 9)
    log(f"[bench] c4: step {ms:.3f} ms, full-layer decode {ms_full * 1e3:.1f} us")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    achieved = bench.full_bytes / (ms_full * 1e-3) / 1e9
    res = dict(
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 4), dtype="bf16",
        config={"workload": "mixed 48-layer decode step B=32, T=32K, 39 SWA (W=128, 8kv) + 9 full (4kv) layers, "
                            "64q, D=128, bf16, page 64, SWA ratio 0.1, one swa_decode_step call",
                "global_batch": st.batch, "seq_len": st.seq_len, "layers": 48},
        tokens_per_s=round(st.batch / (ms * 1e-3), 1),
        frac_of_hbm_peak=round(value / HBM_PEAK_GBS, 4),
        roofline=dict(kernel="swa_decode full layer (split-K + merge)", bound="hbm", achieved=round(achieved, 1),
                      peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_decode_full_c4", DECODE_SRC),
                      bytes_per_launch=bench.full_bytes, us_per_launch=round(ms_full * 1e3, 2),
                      splits=bench.splits, **pct),
    )
    if cpu is not None:
        res["cpu_baseline"] = cpu
    del bench
    torch.cuda.empty_cache()
    return res


# ---------------------------------------------------------------------------
# unified: the c2 decode batch over one unified sub-pool of 32 layers
# ---------------------------------------------------------------------------


class UnifiedBench:
    """The c2 decode step with its 32 SWA layers in one raw buffer of page-major
    envelopes, read through the library's dense per-layer views."""

    def __init__(self, torch, swa, ub, seed=9):
        self.torch, self.swa, self.ub = torch, swa, ub
        B, Hq, Hkv, D, L, P = ub.batch, ub.q_heads, ub.kv_heads, ub.head_dim, ub.layers, ub.page_size
        self.mult = 2 * L
        self.raw_bytes = swa.swa_unified_pool_bytes(L, Hkv, D, torch.bfloat16, P, ub.n_phys)
        self.raw = torch.empty(self.raw_bytes, dtype=torch.uint8, device="cuda")
        g = torch.Generator(device="cuda")
        g.manual_seed(seed)
        flat = self.raw.view(torch.bfloat16)
        chunk = 1 << 26
        for at in range(0, flat.numel(), chunk):
            n = min(chunk, flat.numel() - at)
            flat[at:at + n] = torch.randn(n, generator=g, device="cuda").to(torch.bfloat16)
        self.views = swa.swa_unified_layer_views(self.raw, 0, L, Hkv, D, torch.bfloat16, P, ub.n_phys)
        self.v2p = torch.from_numpy(ub.v2p).cuda()
        self.index = swa.IndexTables(torch.from_numpy(ub.req_to_token).cuda(), torch.from_numpy(ub.req_pool_idx).cuda(),
                                     torch.from_numpy(ub.seq_lens).cuda(), None, P)
        virt = ub.req_to_token[ub.req_pool_idx, ub.seq_lens - 1].astype(np.int64)   # each request's current token
        self.new_virt = torch.from_numpy(virt).cuda()
        self.new_ids = torch.empty_like(self.new_virt)
        self.table = torch.empty(B * (ub.window + 1), dtype=torch.int32, device="cuda")
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        self.sinks = torch.from_numpy(ub.sinks).cuda()
        self.layers = [dict(q=randn_store(torch, (B, Hq, D), g, "bf16"),
                            new_k=randn_store(torch, (B, Hkv, D), g, "bf16"),
                            new_v=randn_store(torch, (B, Hkv, D), g, "bf16"),
                            out=torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")) for _ in range(L)]
        # algorithmic bytes, as for the two-pool decode step (window only), the
        # kernel-id translation reading one page-table entry per position
        n_keys = np.minimum(ub.seq_lens.astype(np.int64), ub.window + 1)
        self.decode_bytes = int(n_keys.sum() * Hkv * D * 2 * 2 + B * Hq * D * 4 + n_keys.sum() * 4 + (B + 1) * 4)
        self.store_bytes = B * Hkv * D * 2 * 2 + B * 8
        self.translate_bytes = B * 8 * 3 + int(n_keys.sum()) * (4 + 8 + 4) + B * 12
        self.step_bytes = self.translate_bytes + L * (self.store_bytes + self.decode_bytes)

    def step(self):
        swa, ub = self.swa, self.ub
        swa.swa_translate_kernel_ids(self.new_virt, self.v2p, ub.page_size, self.mult, self.new_ids)
        swa.swa_translate_window_unified(self.index, self.v2p, self.mult, ub.window, self.table, self.indptr)
        self.dominant()

    def dominant(self):
        swa, ub = self.swa, self.ub
        for view, ly in zip(self.views, self.layers):
            swa.swa_decode_store(ly["q"], view, self.index, ub.window, ly["out"], self.new_ids, ly["new_k"],
                                 ly["new_v"], sinks=self.sinks, slot_table=self.table, table_indptr=self.indptr,
                                 use_map=False)


def run_unified_workload(args, torch, swa, W):
    ub = W.unified_c2_decode()
    log(f"[bench] unified: building one sub-pool of {ub.layers} layers")
    bench = UnifiedBench(torch, swa, ub)
    ms = timed_step(torch, bench.step, args.steps, args.warmup)
    ms_dec, pct = timed_dominant(torch, bench.dominant, max(10, args.steps // 2), ub.layers)
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    dom_bytes = bench.decode_bytes + bench.store_bytes
    achieved = dom_bytes / (ms_dec * 1e-3) / 1e9
    log(f"[bench] unified step {ms:.4f} ms; swa_decode_store {ms_dec * 1e3:.2f} us per layer")
    return dict(
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 5), dtype="bf16",
        config={"workload": "batched SWA decode B=64, T~U[1K,8K], W=128, 64q/8kv, D=128, bf16, page 16, over one "
                            "unified sub-pool of 32 layers (page-major envelopes, dense per-layer views)",
                "global_batch": int(ub.batch), "layers_per_step": ub.layers, "window": ub.window,
                "pool_bytes": int(bench.raw_bytes)},
        tokens_per_s=round(ub.batch / (ms * 1e-3), 1),
        roofline=dict(kernel="swa_decode_store (store fused) over unified views", bound="hbm",
                      achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_decode_unified_c2", DECODE_SRC), bytes_per_launch=dom_bytes,
                      us_per_launch=round(ms_dec * 1e3, 3), **pct),
    )


# ---------------------------------------------------------------------------
# evict: SWA eviction of a batch right after its prefill
# ---------------------------------------------------------------------------


class EvictBench:
    """The after-prefill eviction batch on `copies` distinct copies of its index
    tables (req_to_token, mapping, evicted lengths), so that back-to-back calls
    are not served from the 256 MB Infinity Cache.  A call consumes its copy's
    mapping; restore() puts the pristine mapping back (outside the timed
    events)."""

    def __init__(self, torch, swa, eb, copies=16):
        self.torch, self.swa, self.eb, self.copies = torch, swa, eb, copies
        B, P = eb.batch, eb.page_size
        rows = torch.from_numpy(eb.req_pool_idx).cuda()
        lens = torch.from_numpy(eb.seq_lens).cuda()
        self.pre = torch.from_numpy(eb.pre_lens).cuda()
        self.map0 = torch.from_numpy(eb.full_to_swa).cuda()
        self.ev0 = torch.from_numpy(eb.evicted_lens).cuda()
        self.index = [swa.IndexTables(torch.from_numpy(eb.req_to_token).cuda(), rows, lens, None, P)
                      for _ in range(copies)]
        self.maps = [torch.empty_like(self.map0) for _ in range(copies)]
        self.evs = [torch.empty_like(self.ev0) for _ in range(copies)]
        cap = B * (eb.req_to_token.shape[1] // P + 2)  # at most one report per page plus the first
        self.pages = [torch.empty(cap, dtype=torch.int64, device="cuda") for _ in range(copies)]
        self.count = [torch.zeros(1, dtype=torch.int64, device="cuda") for _ in range(copies)]
        need = swa.lib.swa_evict_workspace_bytes(B, eb.req_to_token.shape[1], P)
        self.ws = torch.empty(need // 4, dtype=torch.int32, device="cuda")
        self.restore()

    def released(self):
        """Positions and pages the last call on copy 0 released (from its
        advanced evicted lengths and its page count)."""
        moved = (self.evs[0].long() - self.ev0.long()).clamp_min(0)
        return int(moved.sum().item()), int(self.count[0].item())

    def restore(self):
        for m, e in zip(self.maps, self.evs):
            m.copy_(self.map0)
            e.copy_(self.ev0)

    def calls(self):
        for i in range(self.copies):
            self.swa.swa_evict(self.index[i], self.maps[i], self.pre, self.evs[i], self.eb.window, self.pages[i],
                               self.count[i], interval=128, workspace=self.ws)


def run_evict_workload(args, torch, swa, W):
    eb = W.evict_after_prefill()
    log("[bench] evict: building 16 copies of the index tables")
    bench = EvictBench(torch, swa, eb)
    g = graph_of(torch, bench.calls)
    for _ in range(max(1, args.warmup // bench.copies)):
        bench.restore()
        g.replay()
    n_rep = max(1, -(-args.steps // bench.copies))
    starts = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep)]
    ends = [torch.cuda.Event(enable_timing=True) for _ in range(n_rep)]
    torch.cuda.synchronize()
    for r in range(n_rep):
        bench.restore()  # untimed: the calls consume their copies' mappings
        starts[r].record()
        g.replay()
        ends[r].record()
    torch.cuda.synchronize()
    per_call = np.array([s.elapsed_time(e) for s, e in zip(starts, ends)]) / bench.copies  # ms
    ms = float(per_call.mean())
    positions, pages = bench.released()
    # a further replay finds every request's interval gate shut: the per-step cost
    # of calling the eviction when nothing is due (skipped in profiling runs)
    noop = None if args.skip_noop else time_replays(torch, g, 20) / bench.copies
    # algorithmic bytes of one call: per released position its req_to_token
    # entry (4 B) and its mapping entry cleared (8 B); per candidate (the range's
    # first position and each page start: here every one reports a page) its
    # mapping entry read (8 B) and the int64 report; per request req_pool_idx,
    # pre_lens and evicted_lens read (12 B) and evicted_lens written (4 B); the
    # count (8 B).
    nbytes = positions * 12 + pages * 16 + eb.batch * 16 + 8
    value = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] evict {ms * 1e3:.2f} us per call, {positions} positions, {pages} pages; "
        f"no-op call {'-' if noop is None else f'{noop * 1e3:.2f}'} us")
    return dict(
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 5), dtype="int64", steps=n_rep * bench.copies,
        config={"workload": "SWA eviction right after prefill: B=256, lognormal lengths (median 16K, clipped to "
                            "[512, 64K]), W=128, page 64, decode interval 128, every position mapped",
                "global_batch": int(eb.batch), "window": eb.window, "page_size": eb.page_size,
                "released_positions": int(positions), "released_pages": pages},
        timed="back-to-back calls on 16 distinct copies of the index tables, replayed as one graph; the "
              "mappings are restored between replays, outside the timed events",
        positions_per_s=round(positions / (ms * 1e-3), 1),
        noop_call_us=None if noop is None else round(noop * 1e3, 3),
        roofline=dict(kernel="swa_evict (scan + apply)", bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS,
                      unit="GB/s", frac=round(value / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_evict_after_prefill", ["evict_kernels.hip", "common.hpp",
                                                                               "api.cpp"]),
                      bytes_per_launch=nbytes, us_per_launch=round(ms * 1e3, 3),
                      p10_us=round(float(np.percentile(per_call, 10)) * 1e3, 3),
                      p50_us=round(float(np.percentile(per_call, 50)) * 1e3, 3),
                      p90_us=round(float(np.percentile(per_call, 90)) * 1e3, 3)),
    )


# ---------------------------------------------------------------------------
# alloc: paired allocation for the c5 batch (a prefill chunk, a decode step)
# ---------------------------------------------------------------------------


class AllocBench:
    """One allocation call on device copies of an allocation state.  The call
    only writes outputs and mapping entries whose values do not depend on what
    the previous call wrote, so replays repeat the same work."""

    def __init__(self, torch, swa, ab, decode):
        self.torch, self.swa, self.ab, self.decode = torch, swa, ab, decode
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()  # noqa: E731
        self.pre, self.seq, self.last = dev(ab.pre_lens), dev(ab.seq_lens), dev(ab.last_loc)
        self.map = dev(ab.full_to_swa)
        self.free_full, self.free_swa = dev(ab.free_full), dev(ab.free_swa)
        self.n = ab.batch if decode else int((ab.seq_lens.astype(np.int64) - ab.pre_lens).sum())
        self.out_full = torch.empty(self.n, dtype=torch.int64, device="cuda")
        self.out_swa = torch.empty(self.n, dtype=torch.int64, device="cuda")
        self.new_pages = torch.zeros(1, dtype=torch.int64, device="cuda")
        self.pages = swa.swa_alloc_pages_needed(None if decode else ab.pre_lens, ab.seq_lens, ab.page_size)
        # algorithmic bytes: per request its lengths and last_loc (16 B, decode 12 B) and
        # the mapped last_loc (8 B); per new position both slots written (16 B) and its
        # mapping entry written (8 B); per new page one entry read from each free list
        self.bytes = ab.batch * ((12 if decode else 16) + 8) + self.n * 24 + self.pages * 16 + 8

    def call(self):
        ab, swa = self.ab, self.swa
        if self.decode:
            ok = swa.swa_alloc_decode(self.seq, self.last, ab.page_size, self.free_full, self.out_full,
                                      free_swa=self.free_swa, full_to_swa=self.map, out_swa=self.out_swa,
                                      new_pages=self.new_pages, seq_lens_host=ab.seq_lens)
        else:
            ok = swa.swa_alloc_extend(self.pre, self.seq, self.last, ab.page_size, self.free_full, self.out_full,
                                      free_swa=self.free_swa, full_to_swa=self.map, out_swa=self.out_swa,
                                      new_pages=self.new_pages, pre_lens_host=ab.pre_lens, seq_lens_host=ab.seq_lens)
        if not ok:
            raise RuntimeError("allocation refused: free lists too short")


def run_alloc_workload(args, torch, swa, W):
    log("[bench] alloc: building the prefill-chunk and decode-step states")
    ext = AllocBench(torch, swa, W.alloc_prefill_chunk(), decode=False)
    dec = AllocBench(torch, swa, W.alloc_decode_step(), decode=True)
    reps = 32  # calls per graph replay
    g_ext = graph_of(torch, lambda: [ext.call() for _ in range(reps)])
    g_dec = graph_of(torch, lambda: [dec.call() for _ in range(reps)])
    for _ in range(max(1, args.warmup // reps)):
        g_ext.replay()
        g_dec.replay()
    n_rep = max(1, -(-args.steps // reps))
    ms = time_replays(torch, g_ext, n_rep) / reps
    pct = replay_percentiles(torch, g_ext, n_rep, reps)
    ms_dec = time_replays(torch, g_dec, n_rep) / reps
    value = ext.bytes / (ms * 1e-3) / 1e9
    log(f"[bench] alloc_extend {ms * 1e3:.2f} us ({ext.n} positions, {ext.pages} pages per pool); "
        f"alloc_decode {ms_dec * 1e3:.2f} us ({dec.n} requests, {dec.pages} pages)")
    return dict(
        value=round(value, 1), unit="GB/s", ms_per_step=round(ms, 5), dtype="int64", steps=n_rep * reps,
        config={"workload": "paired allocation (full and SWA pool, mapping written) of one 2048-position prefill "
                            "chunk for each of 256 requests with lognormal lengths (median 16K), page 64",
                "global_batch": int(ext.ab.batch), "page_size": ext.ab.page_size, "new_positions": ext.n,
                "new_pages_per_pool": int(ext.pages)},
        positions_per_s=round(ext.n / (ms * 1e-3), 1),
        decode_step_us=round(ms_dec * 1e3, 3),
        decode_step="alloc_decode of one position for each of the same 256 requests",
        roofline=dict(kernel="alloc_extend", bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(value / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_alloc_prefill_chunk", ["alloc_kernels.hip", "common.hpp",
                                                                               "api.cpp"]),
                      bytes_per_launch=ext.bytes, us_per_launch=round(ms * 1e3, 3), **pct),
    )


def copy_probe(torch, reps=5):
    """A plain elementwise kernel of known traffic (1 GiB read + 1 GiB written
    per launch), run so that rocprofv3's FETCH_SIZE / WRITE_SIZE counters can
    be scaled to bytes: factor = known bytes / counter bytes."""
    n = 1 << 28
    src = torch.ones(n, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        torch.neg(src, out=dst)
    torch.cuda.synchronize()
    return {"copy_probe": "torch.neg float32", "bytes_read_per_launch": n * 4, "bytes_written_per_launch": n * 4,
            "launches": reps}


# ---------------------------------------------------------------------------


def host_inputs(names):
    """Host-side workloads (numpy; no GPU) and the per-unit counts the CPU
    baselines need."""
    from sliding_window_attention_swa_amd import workloads as W
    hosts = {}
    for n in names:
        if n == "c4":
            st = W.c4_mixed_step()
            hosts[n] = dict(st=st, step_bytes=mixed_bytes(st)[2])
        elif n in ("c1", "c2", "c5") or n.startswith("c2w_"):
            wl, layers, desc = decode_host(n)
            out_dtype = "f32" if wl.q_dtype == "f32" else "bf16"
            dec, store, translate, fused, _ = decode_bytes(wl, out_dtype)
            hosts[n] = dict(wl=wl, layers=layers, desc=desc, layer_bytes=dec + store + translate)
        else:
            window = 128 if n == "c3" else int(n.split("_")[1])
            wl = extend_host(window)
            flops = extend_counts(wl)[0]
            # a call of the oracle decodes the whole chunk's queries first (~0.4 s) and a row
            # costs about W + 1 keys: tasks of ~1 s of rows keep that fixed part small
            hosts[n] = dict(wl=wl, flops_per_row=flops / wl.q.shape[0],
                            rows_per_task=max(16, 512 * 128 // window))
    return hosts


def measure_probes(torch, swa):
    """The practical ceilings next to the published peaks (include/swa_probe.h):
    one streaming read of 2 GiB and one copy of 1 GiB with 16-byte accesses
    (best over grids of 1,024 to 4,096 workgroups) and a loop of nothing but
    bf16 MFMAs (two, four or eight wavefronts per SIMD), each the best of five
    timed launches."""
    def best_ms(fn, reps=5):
        fn()
        torch.cuda.synchronize()
        ms = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record()
            fn()
            e1.record()
            torch.cuda.synchronize()
            ms.append(e0.elapsed_time(e1))
        return min(ms)

    nbytes = 2 << 30
    buf = torch.zeros(nbytes, dtype=torch.uint8, device="cuda")
    read = {}
    for grid in (1024, 2048, 4096):
        out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        read[grid] = nbytes / (best_ms(lambda: swa.swa_probe_read(buf, out, grid)) * 1e-3) / 1e9
    del buf, out
    half = nbytes // 2  # 1 GiB read and 1 GiB written
    src = torch.zeros(half, dtype=torch.uint8, device="cuda")
    dst = torch.empty(half, dtype=torch.uint8, device="cuda")
    copy = {}
    for grid in (1024, 2048, 4096):
        copy[grid] = 2 * half / (best_ms(lambda: swa.swa_probe_copy(src, dst, grid)) * 1e-3) / 1e9
    del src, dst
    mfma, iters = {}, 4096
    for grid in (512, 1024, 2048):
        out = torch.empty(grid * 256, dtype=torch.float32, device="cuda")
        flops = grid * 4 * iters * 8 * 16384
        mfma[grid] = flops / (best_ms(lambda: swa.swa_probe_mfma(out, grid, iters)) * 1e-3) / 1e12
    torch.cuda.empty_cache()
    g_read, g_copy, g_mfma = max(read, key=read.get), max(copy, key=copy.get), max(mfma, key=mfma.get)
    log(f"[bench] probes: read {read[g_read]:.1f} GB/s (grid {g_read}), copy {copy[g_copy]:.1f} GB/s read + written "
        f"(grid {g_copy}), bf16 MFMA {mfma[g_mfma]:.1f} TFLOP/s (grid {g_mfma})")
    return dict(hbm_read_gbs=round(read[g_read], 1), hbm_read_frac_of_peak=round(read[g_read] / HBM_PEAK_GBS, 4),
                hbm_copy_gbs=round(copy[g_copy], 1), hbm_copy_frac_of_peak=round(copy[g_copy] / HBM_PEAK_GBS, 4),
                mfma_bf16_tflops=round(mfma[g_mfma], 1),
                mfma_frac_of_peak=round(mfma[g_mfma] / BF16_PEAK_TFLOPS, 4),
                read="swa_probe_read: one pass over 2 GiB, 16-byte loads, grid-stride",
                copy="swa_probe_copy: 1 GiB read and 1 GiB written, 16-byte loads and stores, grid-stride",
                mfma="swa_probe_mfma: 8 independent v_mfma_f32_16x16x32_bf16 chains per wavefront")


def against_probes(res, probes):
    """Each roofline also as a fraction of the probe that bounds it."""
    roof = res.get("roofline")
    if not roof or not probes:
        return
    if roof.get("unit") == "GB/s":
        roof["frac_of_probe"] = round(roof["achieved"] / probes["hbm_read_gbs"], 4)
        roof["frac_of_copy_probe"] = round(roof["achieved"] / probes["hbm_copy_gbs"], 4)
    elif roof.get("unit") == "TFLOP/s":
        roof["frac_of_probe"] = round(roof["achieved"] / probes["mfma_bf16_tflops"], 4)
    if "tflops" in roof and roof.get("achieved_gbs"):  # an extend: the attainable roofline of the probes
        intensity = roof["tflops"] * 1e3 / roof["achieved_gbs"]  # FLOP per byte
        att = min(probes["mfma_bf16_tflops"], intensity * probes["hbm_read_gbs"] / 1e3)
        roof["attainable_tflops_of_probes"] = round(att, 1)
        roof["frac_of_attainable_of_probes"] = round(roof["tflops"] / att, 4)


def contract_line(args, res, name):
    """The one JSON line of the benchmark contract around a workload result."""
    line = dict(metric=METRIC, value=res["value"], unit=res["unit"], n_gpus=1, steps=res.get("steps", args.steps),
                warmup=args.warmup, ms_per_step=res["ms_per_step"], higher_is_better=True, scaling="weak",
                vs_baseline=None, dtype=res.get("dtype", "bf16"), data="synthetic",
                config=dict(res["config"], parallelism="none (1 GPU)"))
    for k, v in res.items():
        if k not in line and k not in ("steps",):
            line[k] = v
    line["config"]["workload_name"] = name
    return line


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--workload", default="all",
                    choices=["all", "c1", "c2", "c2w", "c3", "c3w", "c4", "c5", "evict", "alloc", "unified"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-noop", action="store_true",
                    help="evict: skip timing the calls that release nothing (for profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a copy kernel of known size (counter calibration)")
    ap.add_argument("--window", type=int, default=None, help="c2w / c3w: one window of the sweep only")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)

    if args.copy_probe:
        names = []
    elif args.workload == "all":
        names = (["c4", "c2", "c5"] + [f"c2w_{w}" for w in DECODE_WINDOWS] + ["c3"]
                 + [f"c3w_{w}" for w in SWEEP_WINDOWS] + ["c1"])
    elif args.workload == "c2w":
        names = [f"c2w_{w}" for w in ((args.window,) if args.window else DECODE_WINDOWS)]
    elif args.workload == "c3w":
        names = [f"c3w_{w}" for w in ((args.window,) if args.window else SWEEP_WINDOWS)]
    elif args.workload in ("c1", "c2", "c3", "c4", "c5"):
        names = [args.workload]
    else:
        names = []
    hosts = host_inputs(names)
    cpu = {} if args.no_cpu_baseline or not names else run_cpu_baselines(names, hosts)

    import torch
    from sliding_window_attention_swa_amd import swa
    from sliding_window_attention_swa_amd import workloads as W
    if not torch.cuda.is_available():
        print(json.dumps({"error": "no GPU visible"}), flush=True)
        sys.exit(1)
    torch.cuda.set_device(0)
    if args.copy_probe:
        print(json.dumps(copy_probe(torch)), flush=True)
        return
    probes = measure_probes(torch, swa)
    if args.workload in ("evict", "alloc", "unified"):
        fn = {"evict": run_evict_workload, "alloc": run_alloc_workload, "unified": run_unified_workload}
        res = fn[args.workload](args, torch, swa, W)
        against_probes(res, probes)
        line = contract_line(args, res, args.workload)
        line["probes"] = probes
        print(json.dumps(line), flush=True)
        return

    results = {}
    for n in names:
        h = hosts[n]
        if n == "c4":
            results[n] = run_mixed_gpu(args, torch, swa, h["st"], cpu.get(n))
        elif n in ("c1", "c2", "c5") or n.startswith("c2w_"):
            results[n] = run_decode_gpu(args, torch, swa, n, h["wl"], h["layers"], h["desc"], cpu.get(n))
        else:
            results[n] = run_extend_gpu(args, torch, swa, n, h["wl"], cpu.get(n))
    for r in results.values():
        against_probes(r, probes)
    head = names[0]
    line = contract_line(args, results[head], head)
    line["probes"] = probes
    if len(names) > 1:
        line["sub_results"] = {n: results[n] for n in names[1:]}
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
