"""Benchmark of the sliding-window attention hot path on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload c2|c1|c3|c4|c5|evict|alloc|unified]

Other workloads (one JSON line each, same fields): c1 single f32 decode; c3
chunked-prefill extend (store + extend over 4 layers); c4 the 48-layer mixed
decode step (39 SWA + 9 full layers); c5 fp8-KV decode with store; evict the
SWA eviction of the c5 batch right after its prefill; alloc the paired
allocation of a prefill chunk (and of a decode step) for the c5 batch;
unified the c2 decode step over one unified sub-pool of 32 layers.

Default workload (c2): batched SWA decode, B = 64 requests with context lengths
uniform in [1K, 8K], W = 128, 64 q / 8 kv heads, head_dim 128, bf16, page 16,
two-pool cache with out-of-window pages tombstoned.  One step is one decode
step of that batch through a stack of 32 SWA layers, each with its own K/V
pool (so the 256 MB Infinity Cache cannot serve repeats):
    translate_loc (new tokens' full locs -> SWA slots)    once per step
    translate_window (req_to_token -> full -> SWA slots)  once per step
    per layer: swa_decode_store (the new token's K/V store fused into the
               windowed decode; equal to kv_store followed by swa_decode)
The step is captured once as a HIP graph and replayed; inputs are resident in
HBM before timing starts.  The JSON line reports algorithmic HBM bytes per
second of the whole step, the dominant kernel's roofline (swa_decode, timed
live with HIP events over back-to-back launches), and the CPU oracle timed on
the host for a bounded sample of the same work.
"""

from __future__ import annotations

import argparse
import hashlib
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0        # MI355X HBM3E, GB/s
BF16_PEAK_TFLOPS = 2500.0    # MI355X dense bf16 MFMA, TFLOP/s
METRIC = "SWA decode HBM GB/s & tokens/s; windowed prefill TFLOP/s (% of MI355X peak)"


def log(msg):
    print(msg, file=sys.stderr, flush=True)


def source_sha(*names) -> str:
    h = hashlib.sha256()
    for n in names:
        with open(os.path.join(ROOT, "sliding_window_attention_swa_amd", "csrc", n), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def traffic_from_profile(name: str, kernel_files, per_launch_units: float):
    """HBM bytes per launch from committed rocprofv3 counter summaries, or None
    when absent or taken on another version of the kernel source."""
    path = os.path.join(ROOT, "profiles", f"{name}_pmc.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        d = json.load(f)
    if d.get("kernel_source_sha") != source_sha(*kernel_files):
        return None
    return d.get("hbm_bytes_per_launch")


# ---------------------------------------------------------------------------
# device setup helpers (torch for memory only)
# ---------------------------------------------------------------------------


def dev_from_bits(torch, bits, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).cuda().view(torch.bfloat16)
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).cuda()
    return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).cuda()


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


class DecodeBench:
    """A decode batch of one workload replicated over `layers` SWA layers."""

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
            self.layers.append(dict(
                kv=swa.KvLayer(k, v),
                q=randn_store(torch, (B, Hq, D), g, wl.q_dtype),
                new_k=randn_store(torch, (B, Hkv, D), g, "bf16" if wl.kv_dtype != "f32" else "f32"),
                new_v=randn_store(torch, (B, Hkv, D), g, "bf16" if wl.kv_dtype != "f32" else "f32"),
                out=torch.empty((B, Hq, D), dtype=torch.bfloat16 if out_dtype == "bf16" else torch.float32,
                                device="cuda"),
            ))
        self.sinks = torch.from_numpy(wl.sinks).cuda() if wl.sinks is not None else None
        # algorithmic bytes (window only): K/V rows, Q, O, window table
        n_keys = np.minimum(wl.seq_lens.astype(np.int64), wl.window + 1)
        kv_b = {"bf16": 2, "e4m3": 1, "f32": 4}[wl.kv_dtype]
        q_b = {"bf16": 2, "f32": 4}[wl.q_dtype]
        o_b = 2 if out_dtype == "bf16" else 4
        self.decode_bytes = int(n_keys.sum() * Hkv * D * kv_b * 2 + B * Hq * D * (q_b + o_b) + n_keys.sum() * 4
                                + (B + 1) * 4)
        new_b = 2 if wl.kv_dtype != "f32" else 4
        # The new token's store is fused into the decode launch (swa_decode_store):
        # its K/V are read once, as the window's last row (counted in
        # decode_bytes), and written once to the pool (counted here).
        # (bf16 pools only: the e4m3 variant needs more registers, which costs
        # a workgroup per CU, more than the separate store launch costs)
        self.fused = self.has_store and wl.kv_dtype == "bf16" and 0 <= wl.window <= 255
        if self.fused:
            self.store_bytes = B * Hkv * D * kv_b * 2 + B * 8
        else:
            self.store_bytes = B * Hkv * D * 2 * (new_b + kv_b) + B * 8 if self.has_store else 0
        self.translate_bytes = (B * 8 * 3 if self.has_store else 0) + int(n_keys.sum()) * (4 + 8 + 4) + B * 12
        self.step_bytes = self.translate_bytes + layers * (self.store_bytes + self.decode_bytes)
        self.flops_decode = int(n_keys.sum()) * Hq * D * 4

    def step(self):
        swa, wl = self.swa, self.wl
        if self.has_store:
            swa.swa_translate_loc(self.full_loc, self.map, self.swa_loc)
        swa.swa_translate_window(self.index, wl.window, self.table, self.indptr)
        for ly in self.layers:
            self.layer_call(ly)

    def layer_call(self, ly):
        swa, wl = self.swa, self.wl
        if self.fused:
            swa.swa_decode_store(ly["q"], ly["kv"], self.index, wl.window, ly["out"], self.swa_loc, ly["new_k"],
                                 ly["new_v"], sinks=self.sinks, slot_table=self.table, table_indptr=self.indptr)
            return
        if self.has_store:
            swa.swa_kv_store(ly["kv"], self.swa_loc, ly["new_k"], ly["new_v"])
        swa.swa_decode(ly["q"], ly["kv"], self.index, wl.window, ly["out"], sinks=self.sinks,
                       slot_table=self.table, table_indptr=self.indptr)

    def dominant(self):
        """Back-to-back decode launches only (one per layer; with the store fused
        in when the step fuses it)."""
        swa, wl = self.swa, self.wl
        for ly in self.layers:
            if self.fused:
                swa.swa_decode_store(ly["q"], ly["kv"], self.index, wl.window, ly["out"], self.swa_loc,
                                     ly["new_k"], ly["new_v"], sinks=self.sinks, slot_table=self.table,
                                     table_indptr=self.indptr)
            else:
                swa.swa_decode(ly["q"], ly["kv"], self.index, wl.window, ly["out"], sinks=self.sinks,
                               slot_table=self.table, table_indptr=self.indptr)


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


# ---------------------------------------------------------------------------
# CPU baseline: the oracle as it stands, single-threaded, on a bounded sample
# ---------------------------------------------------------------------------


def cpu_baseline_decode(wl, budget_s=12.0):
    from threadpoolctl import threadpool_limits
    from oracle import swa_oracle as O
    B = wl.batch
    done_req = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        pk, pv = wl.pool_k, wl.pool_v
        if wl.new_full_loc is not None:
            swa_loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
            pk, pv = O.kv_store(pk, pv, swa_loc, wl.new_k, wl.new_v, wl.new_dtype, wl.kv_dtype)
        O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window)
        b = 0
        while time.perf_counter() - t0 < budget_s:
            only = [(b, h) for h in range(wl.q_heads)]
            O.decode(wl.q, wl.q_dtype, pk, pv, wl.kv_dtype, wl.req_to_token, wl.req_pool_idx, wl.seq_lens,
                     wl.full_to_swa, wl.window, wl.sinks, only=only)
            b = (b + 1) % B
            done_req += 1
    return time.perf_counter() - t0, done_req


# ---------------------------------------------------------------------------


def run_decode_workload(args, torch, swa, W):
    name = args.workload
    if name == "c2":
        wl, layers = W.c2_decode_bf16(), 32
        desc = "batched SWA decode B=64, T~U[1K,8K], W=128, 64q/8kv, D=128, bf16, page 16"
    elif name == "c5":
        wl, layers = W.c5_decode_fp8(), 16
        desc = "fp8 KV decode B=256, T~lognormal(16K), W=128, 64q/8kv, D=128, e4m3 K/V, bf16 q, page 64"
    else:
        wl, layers = W.c1_decode_f32(), 8
        desc = "single SWA decode T=512, W=128, 8q/8kv, D=128, f32, page 1"
    out_dtype = "f32" if wl.q_dtype == "f32" else "bf16"
    log(f"[bench] {name}: building {layers} layers")
    bench = DecodeBench(torch, swa, wl, layers, out_dtype)
    g_step = graph_of(torch, bench.step)
    for _ in range(args.warmup):
        g_step.replay()
    ms = time_replays(torch, g_step, args.steps)
    log(f"[bench] step {ms:.4f} ms")
    g_dec = graph_of(torch, bench.dominant)
    dec_reps = max(10, args.steps // 2)
    ms_dec = time_replays(torch, g_dec, dec_reps) / layers
    pct = replay_percentiles(torch, g_dec, dec_reps, layers)
    log(f"[bench] swa_decode {ms_dec * 1e3:.2f} us per launch")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    dom_bytes = bench.decode_bytes + (bench.store_bytes if bench.fused else 0)
    achieved = dom_bytes / (ms_dec * 1e-3) / 1e9
    traffic = traffic_from_profile(f"swa_decode_{name}", ["decode_kernels.hip", "common.hpp", "api.cpp"], 1)
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype={"c5": "bf16 q / e4m3 kv", "c1": "f32"}.get(name, "bf16"), data="synthetic",
        config={"workload": desc, "global_batch": int(wl.batch), "layers_per_step": layers, "window": wl.window,
                "max_seq_len": int(wl.seq_lens.max()), "parallelism": "none (1 GPU)"},
        tokens_per_s=round(wl.batch / (ms * 1e-3), 1),
        layer_tokens_per_s=round(wl.batch * layers / (ms * 1e-3), 1),
        frac_of_hbm_peak=round(value / HBM_PEAK_GBS, 4),
        roofline=dict(kernel="swa_decode_store (store fused)" if bench.fused else "swa_decode", bound="hbm",
                      achieved=round(achieved, 1), peak=HBM_PEAK_GBS,
                      unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4), traffic=traffic,
                      bytes_per_launch=dom_bytes, us_per_launch=round(ms_dec * 1e3, 3), **pct),
    )
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        secs, nreq = cpu_baseline_decode(wl)
        per_req_bytes = bench.decode_bytes / wl.batch
        res["cpu_baseline"] = dict(value=round(nreq * per_req_bytes / secs / 1e9, 6), unit="GB/s", cores=1,
                                   kind="oracle",
                                   sample=f"one layer: translate + store + window table for all {wl.batch} requests, "
                                          f"then decode of {nreq} requests x {wl.q_heads} heads ({secs:.1f} s)")
    return res


# ---------------------------------------------------------------------------
# c3: chunked-prefill extend
# ---------------------------------------------------------------------------


class ExtendBench:
    """The c3 extend batch replicated over `layers` SWA layers."""

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
        lo = np.maximum(wl.prefix_lens.astype(np.int64) - wl.window, 0)
        self.n_keys = (wl.seq_lens.astype(np.int64) - lo)
        self.cap = int(self.n_keys.sum())
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
        # algorithmic bytes and band-only FLOPs of one extend launch
        self.extend_bytes = int(total_q * Hq * D * 2 * 2 + self.n_keys.sum() * Hkv * D * 2 * 2 + self.cap * 4
                                + (B + 1) * 4 * 2 + B * 4 * 2)
        pairs = 0
        for b in range(B):
            i = np.arange(int(wl.prefix_lens[b]), int(wl.seq_lens[b]))
            pairs += int(np.sum(i - np.maximum(i - wl.window, 0) + 1))
        self.extend_flops = pairs * Hq * D * 4
        self.store_bytes = total_q * Hkv * D * 2 * 2 * 2 + total_q * 8
        self.step_bytes = total_q * 8 * 3 + self.cap * 16 + layers * (self.store_bytes + self.extend_bytes)
        self.step_flops = layers * self.extend_flops

    def step(self):
        swa, wl = self.swa, self.wl
        swa.swa_translate_loc(self.full_loc, self.map, self.swa_loc)
        swa.swa_translate_window(self.index, wl.window, self.table, self.indptr, prefix_lens=self.prefix)
        for ly in self.layers:
            swa.swa_kv_store(ly["kv"], self.swa_loc, ly["new_k"], ly["new_v"])
            swa.swa_extend(ly["q"], self.qo, self.prefix, ly["kv"], self.index, wl.window, ly["out"], sinks=self.sinks,
                           slot_table=self.table, table_indptr=self.indptr)

    def dominant(self):
        swa, wl = self.swa, self.wl
        for ly in self.layers:
            swa.swa_extend(ly["q"], self.qo, self.prefix, ly["kv"], self.index, wl.window, ly["out"], sinks=self.sinks,
                           slot_table=self.table, table_indptr=self.indptr)


def cpu_baseline_extend(wl, budget_s=12.0):
    from threadpoolctl import threadpool_limits
    from oracle import swa_oracle as O
    rows_done = 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        swa_loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
        pk, pv = O.kv_store(wl.pool_k, wl.pool_v, swa_loc, wl.new_k, wl.new_v, "bf16", "bf16")
        O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window,
                       prefix_lens=wl.prefix_lens)
        r = 0
        while time.perf_counter() - t0 < budget_s:
            only = [(r, h) for h in range(wl.q_heads)]
            O.extend(wl.q, "bf16", wl.qo_indptr, wl.prefix_lens, pk, pv, "bf16", wl.req_to_token, wl.req_pool_idx,
                     wl.seq_lens, wl.full_to_swa, wl.window, wl.sinks, only=only)
            r = (r + 997) % wl.q.shape[0]
            rows_done += 1
    return time.perf_counter() - t0, rows_done


def run_extend_workload(args, torch, swa, W):
    wl, layers = W.c3_extend_bf16(), 4
    log(f"[bench] c3: building {layers} layers")
    bench = ExtendBench(torch, swa, wl, layers)
    g_step = graph_of(torch, bench.step)
    for _ in range(args.warmup):
        g_step.replay()
    ms = time_replays(torch, g_step, args.steps)
    g_dom = graph_of(torch, bench.dominant)
    ms_ext = time_replays(torch, g_dom, max(5, args.steps)) / layers
    pct = replay_percentiles(torch, g_dom, max(5, args.steps), layers)
    log(f"[bench] step {ms:.4f} ms, extend {ms_ext * 1e3:.2f} us")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    achieved = bench.extend_bytes / (ms_ext * 1e-3) / 1e9
    tflops = bench.extend_flops / (ms_ext * 1e-3) / 1e12
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic",
        config={"workload": "chunked-prefill extend B=4, prefix 8K + chunk 2K, W=128, 64q/8kv, D=128, bf16, page 64",
                "global_batch": int(wl.batch), "new_tokens": int(wl.q.shape[0]), "layers_per_step": layers,
                "window": wl.window, "parallelism": "none (1 GPU)"},
        tokens_per_s=round(wl.q.shape[0] / (ms * 1e-3) * layers / layers, 1),
        extend_tflops=round(tflops, 2), extend_frac_of_mfma_peak=round(tflops / BF16_PEAK_TFLOPS, 4),
        extend_attainable_tflops=round(min(BF16_PEAK_TFLOPS, bench.extend_flops / bench.extend_bytes * HBM_PEAK_GBS
                                           / 1e3), 1),
        roofline=dict(kernel="swa_extend", bound="hbm", achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_extend_c3", ["extend_kernels.hip", "common.hpp", "api.cpp"], 1),
                      bytes_per_launch=bench.extend_bytes, flops_per_launch=bench.extend_flops,
                      us_per_launch=round(ms_ext * 1e3, 3), **pct),
    )
    if not args.no_cpu_baseline:
        secs, rows = cpu_baseline_extend(wl)
        per_row_flops = bench.extend_flops / wl.q.shape[0]
        res["cpu_baseline"] = dict(value=round(rows * per_row_flops / secs / 1e12, 9), unit="TFLOP/s", cores=1,
                                   kind="oracle", sample=f"translate + store + window table, then {rows} query rows x "
                                                         f"{wl.q_heads} heads ({secs:.1f} s)")
    return res


# ---------------------------------------------------------------------------
# c4: 48-layer mixed decode step (39 SWA + 9 full layers)
# ---------------------------------------------------------------------------


class MixedBench:
    def __init__(self, torch, swa, W):
        self.torch, self.swa = torch, swa
        st = self.st = W.c4_mixed_step()
        B, Hq, D = st.batch, st.q_heads, st.head_dim
        self.r2t = torch.from_numpy(st.req_to_token).cuda()
        self.rows = torch.from_numpy(st.req_pool_idx).cuda()
        self.lens = torch.from_numpy(st.seq_lens).cuda()
        self.map = torch.from_numpy(st.full_to_swa).cuda()
        self.index = swa.IndexTables(self.r2t, self.rows, self.lens, self.map, st.page_size)
        self.table = torch.empty(B * 129, dtype=torch.int32, device="cuda")
        self.indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        self.layers = []
        self.splits, ws_bytes = swa.swa_decode_plan(B, Hq, 4, D, -1, st.seq_len)
        self.ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
        for ly in st.layers:
            q, k, v = W.c4_layer_tensors(st, ly)
            self.layers.append(dict(meta=ly, q=q, kv=swa.KvLayer(k, v),
                                    out=torch.empty((B, Hq, D), dtype=torch.bfloat16, device="cuda")))
        T, W1 = st.seq_len, 129
        self.full_bytes = B * T * 4 * D * 2 * 2 + B * Hq * D * 4 + B * T * 4
        self.swa_bytes = B * W1 * 8 * D * 2 * 2 + B * Hq * D * 4 + B * W1 * 4
        self.step_bytes = 9 * self.full_bytes + 39 * self.swa_bytes + B * W1 * 16
        self.full_flops = B * T * Hq * D * 4

    def layer_call(self, ly):
        swa, m = self.swa, ly["meta"]
        if m["kind"] == "full":
            swa.swa_decode(ly["q"], ly["kv"], self.index, -1, ly["out"], num_splits=self.splits, workspace=self.ws,
                           use_map=False)
        else:
            swa.swa_decode(ly["q"], ly["kv"], self.index, 128, ly["out"], slot_table=self.table,
                           table_indptr=self.indptr)

    def step(self):
        self.swa.swa_translate_window(self.index, 128, self.table, self.indptr)
        for ly in self.layers:
            self.layer_call(ly)

    def dominant(self):
        for ly in self.layers:
            if ly["meta"]["kind"] == "full":
                self.layer_call(ly)


def run_mixed_workload(args, torch, swa, W):
    log("[bench] c4: building 48 layers")
    bench = MixedBench(torch, swa, W)
    g_step = graph_of(torch, bench.step)
    for _ in range(args.warmup):
        g_step.replay()
    ms = time_replays(torch, g_step, args.steps)
    g_dom = graph_of(torch, bench.dominant)
    ms_full = time_replays(torch, g_dom, max(3, args.steps // 2)) / 9
    pct = replay_percentiles(torch, g_dom, max(3, args.steps // 2), 9)
    log(f"[bench] step {ms:.3f} ms, full-layer decode {ms_full * 1e3:.1f} us")
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    achieved = bench.full_bytes / (ms_full * 1e-3) / 1e9
    st = bench.st
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 4), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic",
        config={"workload": "mixed 48-layer decode step B=32, T=32K, 39 SWA (W=128, 8kv) + 9 full (4kv) layers, "
                            "64q, D=128, bf16, page 64, SWA ratio 0.1", "global_batch": st.batch,
                "seq_len": st.seq_len, "layers": 48, "parallelism": "none (1 GPU)"},
        tokens_per_s=round(st.batch / (ms * 1e-3), 1),
        roofline=dict(kernel="swa_decode full layer (split-K + merge)", bound="hbm", achieved=round(achieved, 1),
                      peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic_from_profile("swa_decode_full_c4", ["decode_kernels.hip", "common.hpp", "api.cpp"], 1),
                      bytes_per_launch=bench.full_bytes, us_per_launch=round(ms_full * 1e3, 2),
                      splits=bench.splits, **pct),
    )
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


def cpu_baseline_unified(bench, budget_s=12.0):
    """The oracle over the first layer's view (read back to the host once), on
    as many requests as fit the budget."""
    from threadpoolctl import threadpool_limits
    from oracle import swa_oracle as O
    ub = bench.ub
    raw = bench.raw.cpu().numpy()
    ks, vs = O.unified_views(raw, 0, ub.layers, ub.kv_heads, ub.head_dim, np.uint16, ub.page_size, ub.n_phys)
    m = O.unified_mapping(ub.v2p, ub.page_size, bench.mult)
    q = bench.layers[0]["q"].view(bench.torch.int16).cpu().numpy().view(np.uint16)
    done, b = 0, 0
    t0 = time.perf_counter()
    with threadpool_limits(1):
        while time.perf_counter() - t0 < budget_s:
            O.decode(q, "bf16", ks[0], vs[0], "bf16", ub.req_to_token, ub.req_pool_idx, ub.seq_lens, m, ub.window,
                     ub.sinks, only=[(b, h) for h in range(ub.q_heads)])
            b = (b + 1) % ub.batch
            done += 1
    return time.perf_counter() - t0, done


def run_unified_workload(args, torch, swa, W):
    ub = W.unified_c2_decode()
    log(f"[bench] unified: building one sub-pool of {ub.layers} layers")
    bench = UnifiedBench(torch, swa, ub)
    g_step = graph_of(torch, bench.step)
    for _ in range(args.warmup):
        g_step.replay()
    ms = time_replays(torch, g_step, args.steps)
    g_dec = graph_of(torch, bench.dominant)
    dec_reps = max(10, args.steps // 2)
    ms_dec = time_replays(torch, g_dec, dec_reps) / ub.layers
    pct = replay_percentiles(torch, g_dec, dec_reps, ub.layers)
    value = bench.step_bytes / (ms * 1e-3) / 1e9
    dom_bytes = bench.decode_bytes + bench.store_bytes
    achieved = dom_bytes / (ms_dec * 1e-3) / 1e9
    log(f"[bench] unified step {ms:.4f} ms; swa_decode_store {ms_dec * 1e3:.2f} us per layer")
    traffic = traffic_from_profile("swa_decode_unified_c2", ["decode_kernels.hip", "common.hpp", "api.cpp"], 1)
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=args.steps, warmup=args.warmup,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="bf16",
        data="synthetic",
        config={"workload": "batched SWA decode B=64, T~U[1K,8K], W=128, 64q/8kv, D=128, bf16, page 16, over one "
                            "unified sub-pool of 32 layers (page-major envelopes, dense per-layer views)",
                "global_batch": int(ub.batch), "layers_per_step": ub.layers, "window": ub.window,
                "pool_bytes": int(bench.raw_bytes), "parallelism": "none (1 GPU)"},
        tokens_per_s=round(ub.batch / (ms * 1e-3), 1),
        roofline=dict(kernel="swa_decode_store (store fused) over unified views", bound="hbm",
                      achieved=round(achieved, 1), peak=HBM_PEAK_GBS, unit="GB/s", frac=round(achieved / HBM_PEAK_GBS, 4),
                      traffic=traffic, bytes_per_launch=dom_bytes, us_per_launch=round(ms_dec * 1e3, 3), **pct),
    )
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        secs, nreq = cpu_baseline_unified(bench)
        res["cpu_baseline"] = dict(value=round(nreq * bench.decode_bytes / ub.batch / secs / 1e9, 6), unit="GB/s",
                                   cores=1, kind="oracle",
                                   sample=f"one layer's decode of {nreq} requests x {ub.q_heads} heads over the "
                                          f"unified view ({secs:.1f} s)")
    return res


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


def cpu_baseline_evict(eb, budget_s=12.0):
    from oracle import swa_oracle as O
    reps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        O.evict(eb.req_to_token, eb.req_pool_idx, eb.full_to_swa, eb.pre_lens, eb.evicted_lens, eb.window,
                eb.page_size, interval=128)
        reps += 1
    return time.perf_counter() - t0, reps


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
    # of calling the eviction when nothing is due (skipped in profiling runs, whose
    # per-kernel averages should cover the releasing calls only)
    noop = None if args.skip_noop else time_replays(torch, g, 20) / bench.copies
    # algorithmic bytes of one call: per released position its req_to_token
    # entry (4 B) and its mapping entry read and cleared (8 + 8 B); per released
    # page one int64 report; per request req_pool_idx, pre_lens and evicted_lens
    # read (12 B) and evicted_lens written (4 B); the count (8 B).
    nbytes = positions * 20 + pages * 8 + eb.batch * 16 + 8
    value = nbytes / (ms * 1e-3) / 1e9
    log(f"[bench] evict {ms * 1e3:.2f} us per call, {positions} positions, {pages} pages; "
        f"no-op call {'-' if noop is None else f'{noop * 1e3:.2f}'} us")
    traffic = traffic_from_profile("swa_evict_after_prefill", ["evict_kernels.hip", "common.hpp", "api.cpp"], 1)
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=n_rep * bench.copies,
        warmup=args.warmup, ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None,
        dtype="int64", data="synthetic",
        config={"workload": "SWA eviction right after prefill: B=256, lognormal lengths (median 16K, clipped to "
                            "[512, 64K]), W=128, page 64, decode interval 128, every position mapped",
                "global_batch": int(eb.batch), "window": eb.window, "page_size": eb.page_size,
                "released_positions": int(positions), "released_pages": pages,
                "parallelism": "none (1 GPU)"},
        timed="back-to-back calls on 16 distinct copies of the index tables, replayed as one graph; the "
              "mappings are restored between replays, outside the timed events",
        positions_per_s=round(positions / (ms * 1e-3), 1),
        noop_call_us=None if noop is None else round(noop * 1e3, 3),
        roofline=dict(kernel="swa_evict (scan + apply)", bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS,
                      unit="GB/s", frac=round(value / HBM_PEAK_GBS, 4), traffic=traffic, bytes_per_launch=nbytes,
                      us_per_launch=round(ms * 1e3, 3),
                      p10_us=round(float(np.percentile(per_call, 10)) * 1e3, 3),
                      p50_us=round(float(np.percentile(per_call, 50)) * 1e3, 3),
                      p90_us=round(float(np.percentile(per_call, 90)) * 1e3, 3)),
    )
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        secs, reps = cpu_baseline_evict(eb)
        res["cpu_baseline"] = dict(value=round(reps * nbytes / secs / 1e9, 6), unit="GB/s", cores=1, kind="oracle",
                                   sample=f"the whole batch, {reps} times ({secs:.1f} s)")
    return res


# ---------------------------------------------------------------------------
# alloc: paired allocation for the c5 batch (a prefill chunk, a decode step)
# ---------------------------------------------------------------------------


class AllocBench:
    """One allocation call on device copies of an allocation state.  The call
    only writes outputs and mapping entries whose values do not depend on what
    the previous call wrote, so replays repeat the same work."""

    def __init__(self, torch, swa, ab, decode):
        self.torch, self.swa, self.ab, self.decode = torch, swa, ab, decode
        dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
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


def cpu_baseline_alloc(ab, decode, budget_s=12.0):
    from oracle import swa_oracle as O
    reps = 0
    t0 = time.perf_counter()
    while time.perf_counter() - t0 < budget_s:
        O.alloc_paired(ab.pre_lens, ab.seq_lens, ab.last_loc, ab.free_full, ab.free_swa, ab.full_to_swa,
                       ab.page_size, decode=decode)
        reps += 1
    return time.perf_counter() - t0, reps


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
    traffic = traffic_from_profile("swa_alloc_prefill_chunk", ["alloc_kernels.hip", "common.hpp", "api.cpp"], 1)
    res = dict(
        metric=METRIC, value=round(value, 1), unit="GB/s", n_gpus=1, steps=n_rep * reps, warmup=args.warmup,
        ms_per_step=round(ms, 5), higher_is_better=True, scaling="weak", vs_baseline=None, dtype="int64",
        data="synthetic",
        config={"workload": "paired allocation (full and SWA pool, mapping written) of one 2048-position prefill "
                            "chunk for each of 256 requests with lognormal lengths (median 16K), page 64",
                "global_batch": int(ext.ab.batch), "page_size": ext.ab.page_size, "new_positions": ext.n,
                "new_pages_per_pool": int(ext.pages), "parallelism": "none (1 GPU)"},
        positions_per_s=round(ext.n / (ms * 1e-3), 1),
        decode_step_us=round(ms_dec * 1e3, 3),
        decode_step="alloc_decode of one position for each of the same 256 requests",
        roofline=dict(kernel="alloc_extend", bound="hbm", achieved=round(value, 1), peak=HBM_PEAK_GBS, unit="GB/s",
                      frac=round(value / HBM_PEAK_GBS, 4), traffic=traffic, bytes_per_launch=ext.bytes,
                      us_per_launch=round(ms * 1e3, 3), **pct),
    )
    if not args.no_cpu_baseline:
        log("[bench] timing the CPU oracle")
        secs, n = cpu_baseline_alloc(ext.ab, False)
        res["cpu_baseline"] = dict(value=round(n * ext.bytes / secs / 1e9, 6), unit="GB/s", cores=1, kind="oracle",
                                   sample=f"the whole prefill-chunk allocation, {n} times ({secs:.1f} s)")
    return res


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


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=500)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--workload", default="c2", choices=["c1", "c2", "c3", "c4", "c5", "evict", "alloc", "unified"])
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--skip-noop", action="store_true",
                    help="evict: skip timing the calls that release nothing (for profiling runs)")
    ap.add_argument("--copy-probe", action="store_true",
                    help="run only a copy kernel of known size (counter calibration)")
    args = ap.parse_args()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}), flush=True)
        sys.exit(2)
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
    if args.workload == "c3":
        res = run_extend_workload(args, torch, swa, W)
    elif args.workload == "c4":
        res = run_mixed_workload(args, torch, swa, W)
    elif args.workload == "evict":
        res = run_evict_workload(args, torch, swa, W)
    elif args.workload == "alloc":
        res = run_alloc_workload(args, torch, swa, W)
    elif args.workload == "unified":
        res = run_unified_workload(args, torch, swa, W)
    else:
        res = run_decode_workload(args, torch, swa, W)
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
