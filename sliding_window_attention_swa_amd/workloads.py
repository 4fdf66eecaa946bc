"""Seeded synthetic inputs for the five workloads (and scaled-down variants).

This module only draws random numbers and lays out index structures: page
permutations, req_to_token rows, full_to_swa entries, pool contents.  It holds
none of the attention / translation / store arithmetic, and it serves both the
HIP path (tests, benchmark) and the CPU oracle.

Recipe (shared by every workload):
  * independent streams from numpy.random.SeedSequence(seed).spawn(8), used in
    this order: lengths, full pages, SWA pages, Q, K, V, sinks, new K/V;
  * values are float32 N(0, 1) draws rounded to the storage dtype by torch's
    dtype casts (bf16 round-to-nearest-even; e4m3fn: nearest, ties to even);
  * request b lives in req_to_token row b + 1 (row 0 is padding); its
    positions fill pages taken in order from a seeded permutation of the full
    pool's pages 1..N_full/P (page 0 is padding); SWA pages come the same way
    from a permutation of 1..N_swa/P, only for pages that are still live;
  * a position j on full page f (offset k) maps to SWA slot s * P + k when its
    page is live on SWA page s, else to 0 (tombstone);
  * every pool row that no position references, and page 0, holds NaN (e4m3:
    the NaN code 0x7F), so any stray read shows up in the output.
"""

from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import numpy as np
import torch

NAN_BITS = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}
NP_STORE = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}


def to_store(x: np.ndarray, dtype: str) -> np.ndarray:
    """float32 draws -> storage bits of dtype via torch's casts."""
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    if dtype == "f32":
        return t.numpy().copy()
    if dtype == "bf16":
        return t.to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16).copy()
    if dtype == "e4m3":
        return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    raise ValueError(dtype)


class SparsePool:
    """A pool of shape (rows, heads, dim) given by its referenced rows; every
    other row reads as NaN.  Indexing with an integer array returns those rows.
    Used where a dense host copy of a large pool would be wasteful."""

    def __init__(self, rows: int, heads: int, dim: int, dtype: str, used_rows: np.ndarray, values: np.ndarray):
        self.shape = (rows, heads, dim)
        self.dtype = dtype
        order = np.argsort(used_rows, kind="stable")
        self.used_rows = np.asarray(used_rows, dtype=np.int64)[order]
        self.values = values[order]

        self.overlay = {}  # rows written after construction (slot -> row values)

    def __getitem__(self, slots):
        scalar = np.ndim(slots) == 0
        slots = np.atleast_1d(np.asarray(slots, dtype=np.int64))
        out = np.full(slots.shape + self.shape[1:], NAN_BITS[self.dtype], dtype=NP_STORE[self.dtype])
        if len(self.used_rows):
            pos = np.searchsorted(self.used_rows, slots)
            pos_c = np.minimum(pos, len(self.used_rows) - 1)
            hit = (pos < len(self.used_rows)) & (self.used_rows[pos_c] == slots)
            out[hit] = self.values[pos_c[hit]]
        for n, sl in enumerate(slots.tolist()):
            if sl in self.overlay:
                out[n] = self.overlay[sl]
        return out[0] if scalar else out

    def __setitem__(self, slot, row):
        self.overlay[int(slot)] = np.asarray(row, dtype=NP_STORE[self.dtype]).reshape(self.shape[1:])

    def copy(self) -> "SparsePool":
        c = SparsePool.__new__(SparsePool)
        c.shape, c.dtype, c.used_rows, c.values = self.shape, self.dtype, self.used_rows, self.values
        c.overlay = dict(self.overlay)
        return c

    def written_rows(self) -> np.ndarray:
        """Every row that holds a value (initial rows and overlay), sorted."""
        return np.union1d(self.used_rows, np.fromiter(self.overlay.keys(), dtype=np.int64))

    def dense(self) -> np.ndarray:
        out = np.full(self.shape, NAN_BITS[self.dtype], dtype=NP_STORE[self.dtype])
        out[self.used_rows] = self.values
        for sl, row in self.overlay.items():
            out[sl] = row
        return out


@dataclass
class Workload:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    page_size: int
    q_dtype: str
    kv_dtype: str
    seq_lens: np.ndarray                 # int32 (B,)
    req_to_token: np.ndarray             # int32 (B + 1, stride)
    req_pool_idx: np.ndarray             # int32 (B,)
    full_to_swa: Optional[np.ndarray]    # int64 (N_full + P + 1,) or None (single pool / full layer)
    n_full: int
    n_swa: int
    pool_k: SparsePool
    pool_v: SparsePool
    q: np.ndarray                        # storage bits (total_q, Hq, D)
    sinks: Optional[np.ndarray]          # float32 (Hq,) or None
    prefix_lens: Optional[np.ndarray] = None   # extend: int32 (B,)
    qo_indptr: Optional[np.ndarray] = None     # extend: int32 (B + 1,)
    new_full_loc: Optional[np.ndarray] = None  # store: int64 full locs of the new tokens
    new_k: Optional[np.ndarray] = None         # store: (n, Hkv, D) bits of new_dtype
    new_v: Optional[np.ndarray] = None
    new_dtype: str = "bf16"
    ratio: float = 0.8
    notes: dict = field(default_factory=dict)

    @property
    def pool_rows(self) -> int:
        return self.pool_k.shape[0]


def _streams(seed: int):
    return [np.random.default_rng(s) for s in np.random.SeedSequence(seed).spawn(8)]


def _layout(seq_lens, P, n_full, n_swa, live_from_pos, rng_full, rng_swa, stride=None):
    """req_to_token rows and the page-consistent full_to_swa table.

    live_from_pos[b]: positions >= this value (rounded down to its page) keep
    an SWA page; earlier pages are tombstoned."""
    B = len(seq_lens)
    stride = stride or int(max(seq_lens))
    full_pages = rng_full.permutation(np.arange(1, n_full // P + 1, dtype=np.int64))
    swa_pages = rng_swa.permutation(np.arange(1, n_swa // P + 1, dtype=np.int64)) if n_swa else None
    r2t = np.zeros((B + 1, stride), dtype=np.int32)
    mapping = np.zeros(n_full + P + 1, dtype=np.int64)
    mapping[-1] = -1
    fi = si = 0
    swa_rows = []  # (b, position) -> swa slot for referenced positions
    for b, T in enumerate(seq_lens):
        T = int(T)
        npg = -(-T // P)
        fp = full_pages[fi:fi + npg]
        fi += npg
        if fi > len(full_pages):
            raise ValueError("full pool too small for the requests")
        pos = np.arange(T)
        full = fp[pos // P] * P + pos % P
        r2t[b + 1, :T] = full
        if swa_pages is not None:
            first_live = max(0, int(live_from_pos[b])) // P
            live = np.arange(first_live, npg)
            sp = swa_pages[si:si + len(live)]
            si += len(live)
            if si > len(swa_pages):
                raise ValueError("SWA pool too small for the live windows")
            page_to_swa = np.zeros(npg, dtype=np.int64)
            page_to_swa[live] = sp
            mapped = page_to_swa[pos // P]
            slots = np.where(mapped > 0, mapped * P + pos % P, 0)
            mapping[full] = slots
            swa_rows.append(slots)
        else:
            swa_rows.append(full)
    return r2t, mapping, swa_rows


def _fill_pool(rows, H, D, dtype, slot_lists, rng_k, rng_v):
    """Pool rows referenced by any position get N(0,1) values (drawn in
    request / position order); returns two SparsePools."""
    used = np.concatenate([s[s > 0] for s in slot_lists]) if slot_lists else np.zeros(0, np.int64)
    if np.unique(used).size != used.size:
        raise ValueError("two positions share a pool row")
    kv = to_store(rng_k.standard_normal((used.size, H, D), dtype=np.float32), dtype)
    vv = to_store(rng_v.standard_normal((used.size, H, D), dtype=np.float32), dtype)
    return SparsePool(rows, H, D, dtype, used, kv), SparsePool(rows, H, D, dtype, used, vv)


def round_up(x: int, m: int) -> int:
    return -(-x // m) * m


def decode_workload(name, seed, seq_lens, q_heads, kv_heads, window, page_size, q_dtype, kv_dtype, sinks=True,
                    ratio=0.8, live_margin=0, with_store=False, head_dim=128, slack_pages=2, swa_tokens=None,
                    two_pools=True):
    """A batch of decode requests against one SWA layer (window >= 0) of a two-pool
    cache, or against a single full pool (window < 0, or two_pools=False: the
    windowed single-pool mode; positions read from req_to_token directly, no
    SWA pool)."""
    r_len, r_full, r_swa, r_q, r_k, r_v, r_s, r_new = _streams(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B, P = len(seq_lens), page_size
    n_full = round_up(int(sum(round_up(int(t), P) for t in seq_lens)) + slack_pages * P, P)
    use_swa = window >= 0 and two_pools
    if use_swa:
        live_from = np.maximum(seq_lens - 1 - window - live_margin, 0)
        need = int(sum(round_up(int(t), P) - (int(lf) // P) * P for t, lf in zip(seq_lens, live_from)))
        n_swa = swa_tokens or max(round_up(int(math.floor(ratio * n_full)), P), round_up(need + slack_pages * P, P))
        n_swa = n_swa // P * P
    else:
        live_from = np.zeros(B, np.int64)
        n_swa = 0
    r2t, mapping, slot_lists = _layout(seq_lens, P, n_full, n_swa, live_from, r_full, r_swa)
    rows = (n_swa if use_swa else n_full) + P
    pk, pv = _fill_pool(rows, kv_heads, head_dim, kv_dtype, slot_lists, r_k, r_v)
    q = to_store(r_q.standard_normal((B, q_heads, head_dim), dtype=np.float32), q_dtype)
    s = r_s.standard_normal(q_heads).astype(np.float32) if sinks else None
    wl = Workload(name, B, q_heads, kv_heads, head_dim, window, P, q_dtype, kv_dtype, seq_lens.astype(np.int32), r2t,
                  np.arange(1, B + 1, dtype=np.int32), mapping if use_swa else None, n_full, n_swa, pk, pv, q, s,
                  ratio=ratio)
    if with_store:
        # the current token (position T-1) gets new K/V, stored before attention
        wl.new_full_loc = r2t[np.arange(1, B + 1), seq_lens - 1].astype(np.int64)
        wl.new_k = to_store(r_new.standard_normal((B, kv_heads, head_dim), dtype=np.float32), "bf16")
        wl.new_v = to_store(r_new.standard_normal((B, kv_heads, head_dim), dtype=np.float32), "bf16")
        wl.new_dtype = "bf16"
    return wl


def extend_workload(name, seed, prefix_lens, chunk_lens, q_heads, kv_heads, window, page_size, sinks=True,
                    ratio=0.8, head_dim=128, slack_pages=2, two_pools=True, live_from=None):
    """Chunked prefill: each request has a cached prefix whose pages before
    prefix - W (or live_from) are tombstoned on the SWA side, plus a chunk of
    new tokens whose K/V are provided as new_k / new_v (to be stored at
    translate(new_full_loc)).  two_pools=False: one full pool, no mapping (the
    windowed single-pool mode)."""
    r_len, r_full, r_swa, r_q, r_k, r_v, r_s, r_new = _streams(seed)
    prefix = np.asarray(prefix_lens, dtype=np.int64)
    chunk = np.asarray(chunk_lens, dtype=np.int64)
    seq = prefix + chunk
    B, P = len(seq), page_size
    n_full = round_up(int(sum(round_up(int(t), P) for t in seq)) + slack_pages * P, P)
    if live_from is None:
        live_from = np.maximum(prefix - window, 0) if window >= 0 else np.zeros(B, np.int64)
    live_from = np.asarray(live_from, dtype=np.int64)
    need = int(sum(round_up(int(t), P) - (int(lf) // P) * P for t, lf in zip(seq, live_from)))
    n_swa = max(round_up(int(math.floor(ratio * n_full)), P), round_up(need + slack_pages * P, P)) if two_pools else 0
    r2t, mapping, slot_lists = _layout(seq, P, n_full, n_swa, live_from, r_full, r_swa)
    rows = (n_swa if two_pools else n_full) + P
    # pool holds the live prefix window only; chunk rows start as NaN and are stored
    prefix_slots = [s[:int(p)] for s, p in zip(slot_lists, prefix)]
    pk, pv = _fill_pool(rows, kv_heads, head_dim, "bf16", prefix_slots, r_k, r_v)
    total = int(chunk.sum())
    q = to_store(r_q.standard_normal((total, q_heads, head_dim), dtype=np.float32), "bf16")
    s = r_s.standard_normal(q_heads).astype(np.float32) if sinks else None
    qo = np.zeros(B + 1, dtype=np.int32)
    qo[1:] = np.cumsum(chunk)
    new_loc = np.concatenate([r2t[b + 1, int(prefix[b]):int(seq[b])] for b in range(B)]).astype(np.int64)
    wl = Workload(name, B, q_heads, kv_heads, head_dim, window, P, "bf16", "bf16", seq.astype(np.int32), r2t,
                  np.arange(1, B + 1, dtype=np.int32), mapping if two_pools else None, n_full, n_swa, pk, pv, q, s,
                  prefix_lens=prefix.astype(np.int32), qo_indptr=qo, ratio=ratio)
    wl.new_full_loc = new_loc
    wl.new_k = to_store(r_new.standard_normal((total, kv_heads, head_dim), dtype=np.float32), "bf16")
    wl.new_v = to_store(r_new.standard_normal((total, kv_heads, head_dim), dtype=np.float32), "bf16")
    return wl


# ---------------------------------------------------------------------------
# The five workloads at their stated sizes
# ---------------------------------------------------------------------------

SEED_BASE = 20261202


def c1_decode_f32(seed=SEED_BASE + 1) -> Workload:
    """Single SWA layer decode: 1 request, T = 512, W = 128, 8 q / 8 kv heads,
    D = 128, f32, P = 1; positions < T - W - 128 evicted (mapping 0)."""
    T, W = 512, 128
    # live_from = i - W - margin = T - W - 128 with i = T - 1
    return decode_workload("c1_decode_f32_T512", seed, [T], 8, 8, W, 1, "f32", "f32", ratio=0.5, live_margin=127,
                           slack_pages=512, swa_tokens=512)


def c2_decode_bf16(seed=SEED_BASE + 2, batch=64, q_heads=64, kv_heads=8, window=128) -> Workload:
    """Batched SWA decode: B = 64, T ~ U[1024, 8192], W = 128, 64 q / 8 kv heads,
    D = 128, bf16, P = 16, out-of-window pages tombstoned, ratio 0.8.  Other
    windows give the same batch with a longer window (1023 and 4095 keys: the
    long-window layers, split over their keys)."""
    lens = np.random.default_rng(np.random.SeedSequence(seed).spawn(8)[0]).integers(1024, 8193, size=batch)
    name = "c2_decode_bf16_B64" + ("" if window == 128 else f"_W{window}")
    return decode_workload(name, seed, lens, q_heads, kv_heads, window, 16, "bf16", "bf16", ratio=0.8,
                           with_store=True)


def c3_extend_bf16(seed=SEED_BASE + 3, batch=4, prefix=8192, chunk=2048, window=128) -> Workload:
    """Chunked-prefill extend: B = 4, prefix 8K + chunk 2K, W = 128, 64 q / 8 kv
    heads, D = 128, bf16, P = 64; the chunk's K/V are stored first.  Other
    windows give the same shape with a longer band (the prefill window sweep)."""
    name = "c3_extend_bf16_B4_8K+2K" + ("" if window == 128 else f"_W{window}")
    return extend_workload(name, seed, [prefix] * batch, [chunk] * batch, 64, 8, window, 64)


def c5_lengths(seed, batch):
    rng = np.random.default_rng(np.random.SeedSequence(seed).spawn(8)[0])
    return np.clip(np.round(np.exp(rng.normal(math.log(16384), 1.0, size=batch))), 512, 65536).astype(np.int64)


def c5_decode_fp8(seed=SEED_BASE + 5, batch=256, ratio=0.02) -> Workload:
    """fp8 KV decode: B = 256, lognormal lengths (median 16K, sigma 1, clipped to
    [512, 64K]), W = 128, 64 q / 8 kv heads, D = 128, e4m3 K/V (scale 1), bf16 q,
    P = 64, plus a store of one new token per request.  SWA ratio 0.02: every
    live window fits, and a 0.8 pool (~11 GB per layer) would only add NaN rows."""
    lens = c5_lengths(seed, batch)
    return decode_workload("c5_decode_fp8_B256", seed, lens, 64, 8, 128, 64, "bf16", "e4m3", ratio=ratio,
                           with_store=True)


# ---------------------------------------------------------------------------
# Long-context mixed-layer decode step (48 layers) — index structures on the
# host, per-layer K/V drawn on the device from per-layer seeds.
# ---------------------------------------------------------------------------

@dataclass
class MixedStep:
    batch: int
    seq_len: int
    q_heads: int
    head_dim: int
    page_size: int
    layers: List[dict]            # {"id", "kind": "full"|"swa", "window", "kv_heads", "seed"}
    req_to_token: np.ndarray
    req_pool_idx: np.ndarray
    seq_lens: np.ndarray
    full_to_swa: np.ndarray
    n_full: int
    n_swa: int
    swa_slots: np.ndarray         # SWA slots referenced by live windows (to receive values)
    seed: int
    ratio: float
    cell_bytes: float = 0.0


def c4_mixed_step(seed=SEED_BASE + 4, batch=32, seq_len=32768, n_layers=48, full_every=5, n_full_layers=9,
                  ratio=0.1) -> MixedStep:
    """B = 32, T = 32K; 48 layers: 9 full (W = -1, 4 kv heads) at ids 0, 5, ..,
    40 and 39 SWA (W = 128, 8 kv heads); 64 q heads, D = 128, bf16, P = 64; SWA
    pool at ratio 0.1 of the full pool (cell formula); SWA pages live for the
    window plus one eviction interval (128 tokens); no sink."""
    P, W, D = 64, 128, 128
    r_len, r_full, r_swa, *_ = _streams(seed)
    lens = np.full(batch, seq_len, dtype=np.int64)
    n_full = batch * seq_len
    F, S = 4 * (D + D) * 2, 8 * (D + D) * 2
    n_swa = int(math.floor(ratio * n_full)) // P * P
    live_from = lens - 1 - W - 128
    r2t, mapping, slot_lists = _layout(lens, P, n_full, n_swa, live_from, r_full, r_swa)
    full_ids = [full_every * i for i in range(n_full_layers)]
    layers = []
    children = np.random.SeedSequence(seed).spawn(8 + n_layers)[8:]
    for lid in range(n_layers):
        kind = "full" if lid in full_ids else "swa"
        layers.append({"id": lid, "kind": kind, "window": -1 if kind == "full" else W,
                       "kv_heads": 4 if kind == "full" else 8,
                       "seed": int(children[lid].generate_state(1)[0])})
    swa_slots = np.concatenate([s[s > 0] for s in slot_lists])
    return MixedStep(batch, seq_len, 64, D, P, layers, r2t, np.arange(1, batch + 1, dtype=np.int32),
                     lens.astype(np.int32), mapping, n_full, n_swa, swa_slots, seed, ratio,
                     F * n_full_layers + ratio * S * (n_layers - n_full_layers))


def c4_layer_tensors(step: MixedStep, layer: dict, device="cuda"):
    """Per-layer device tensors of the mixed step, drawn from the layer's seed
    with torch's generator on `device`: Q (B, Hq, D) bf16 and the layer's K/V
    pool (rows, Hkv, D) bf16.  Full layers reference every full-pool row; SWA
    layers hold values at the live window slots and NaN elsewhere."""
    g = torch.Generator(device=device)
    g.manual_seed(layer["seed"])
    H, D = layer["kv_heads"], step.head_dim
    q = torch.randn((step.batch, step.q_heads, D), generator=g, device=device).to(torch.bfloat16)
    if layer["kind"] == "full":
        rows = step.n_full + step.page_size
        k = torch.empty((rows, H, D), dtype=torch.bfloat16, device=device)
        v = torch.empty((rows, H, D), dtype=torch.bfloat16, device=device)
        for t, name in ((k, "k"), (v, "v")):
            chunk = 1 << 18
            for r0 in range(0, rows, chunk):
                r1 = min(rows, r0 + chunk)
                t[r0:r1] = torch.randn((r1 - r0, H, D), generator=g, device=device).to(torch.bfloat16)
            t[:step.page_size] = float("nan")  # page 0 is the padding sink
        return q, k, v
    rows = step.n_swa + step.page_size
    k = torch.full((rows, H, D), float("nan"), dtype=torch.bfloat16, device=device)
    v = torch.full((rows, H, D), float("nan"), dtype=torch.bfloat16, device=device)
    idx = torch.from_numpy(step.swa_slots).to(device)
    k[idx] = torch.randn((idx.numel(), H, D), generator=g, device=device).to(torch.bfloat16)
    v[idx] = torch.randn((idx.numel(), H, D), generator=g, device=device).to(torch.bfloat16)
    return q, k, v


# ---------------------------------------------------------------------------
# SWA eviction: index structures only (eviction touches no K/V)
# ---------------------------------------------------------------------------

@dataclass
class EvictBatch:
    name: str
    batch: int
    page_size: int
    window: int
    seq_lens: np.ndarray          # int32 (B,)
    pre_lens: np.ndarray          # int32 (B,): seq_len - 1, the decode position
    evicted_lens: np.ndarray      # int32 (B,)
    req_to_token: np.ndarray      # int32 (B + 1, stride), row 0 padding
    req_pool_idx: np.ndarray      # int32 (B,)
    full_to_swa: np.ndarray       # int64 (n_full + P + 1,), trailing -1 sentinel
    n_full: int
    n_swa: int


def evict_batch(name, seed, seq_lens, page_size, window, live_from=None, evicted_lens=None) -> EvictBatch:
    """A batch whose positions >= live_from (rounded down to a page; default 0,
    i.e. every position) still hold SWA slots, laid out by the same recipe as
    the decode workloads."""
    _, r_full, r_swa, *_ = _streams(seed)
    seq_lens = np.asarray(seq_lens, dtype=np.int64)
    B, P = len(seq_lens), page_size
    live_from = np.zeros(B, np.int64) if live_from is None else np.asarray(live_from, np.int64)
    n_full = round_up(int(sum(round_up(int(t), P) for t in seq_lens)) + 2 * P, P)
    need = int(sum(round_up(int(t), P) - (int(lf) // P) * P for t, lf in zip(seq_lens, live_from)))
    n_swa = round_up(need + 2 * P, P)
    r2t, mapping, _ = _layout(seq_lens, P, n_full, n_swa, live_from, r_full, r_swa)
    ev = np.zeros(B, np.int32) if evicted_lens is None else np.asarray(evicted_lens, np.int32)
    return EvictBatch(name, B, P, window, seq_lens.astype(np.int32), (seq_lens - 1).astype(np.int32), ev, r2t,
                      np.arange(1, B + 1, dtype=np.int32), mapping, n_full, n_swa)


def evict_after_prefill(seed=SEED_BASE + 5, batch=256) -> EvictBatch:
    """The fp8 decode batch (B = 256, lognormal lengths, median 16K, clipped to
    [512, 64K], W = 128, P = 64) right after its prefill: every position still
    holds an SWA slot and nothing has been evicted, so the first decode step's
    eviction releases every page before the window."""
    return evict_batch("evict_after_prefill_B256", seed, c5_lengths(seed, batch), 64, 128)


# ---------------------------------------------------------------------------
# Allocation: index structures and free lists only
# ---------------------------------------------------------------------------

@dataclass
class AllocBatch:
    name: str
    batch: int
    page_size: int
    pre_lens: np.ndarray          # int32 (B,): positions already held
    seq_lens: np.ndarray          # int32 (B,): positions after the allocation
    last_loc: np.ndarray          # int64 (B,): full slot of position pre - 1, or -1
    req_to_token: np.ndarray      # int32 (B + 1, stride)
    req_pool_idx: np.ndarray      # int32 (B,)
    full_to_swa: np.ndarray       # int64 (n_full + P + 1,)
    free_full: np.ndarray         # int64 full pages not in use, in a seeded order
    free_swa: np.ndarray          # int64 SWA pages not in use, in a seeded order
    n_full: int
    n_swa: int


def alloc_batch(name, seed, pre_lens, seq_lens, page_size, window=128, margin=128, slack_pages=4) -> AllocBatch:
    """Requests holding pre_lens positions (laid out like the decode workloads:
    SWA pages only from pre - window - margin on) that will grow to seq_lens;
    both pools get room for the growth plus slack_pages, and every page not in
    use goes on a free list in a seeded order."""
    _, r_full, r_swa, _, _, _, _, r_free = _streams(seed)
    pre = np.asarray(pre_lens, dtype=np.int64)
    seq = np.asarray(seq_lens, dtype=np.int64)
    B, P = len(pre), page_size
    grow = int(sum(-(-int(s) // P) - -(-int(p) // P) for p, s in zip(pre, seq))) * P
    n_full = round_up(int(sum(round_up(int(t), P) for t in pre)) + grow + slack_pages * P, P)
    live_from = np.maximum(pre - window - margin, 0)
    need = int(sum(round_up(int(t), P) - (int(lf) // P) * P for t, lf in zip(pre, live_from)))
    n_swa = round_up(need + grow + slack_pages * P, P)
    r2t, mapping, _ = _layout(pre, P, n_full, n_swa, live_from, r_full, r_swa, stride=max(int(seq.max()), 1))
    used_full = np.unique(r2t[1:][r2t[1:] > 0] // P) if pre.sum() else np.zeros(0, np.int64)
    used_swa = np.unique(mapping[:-1][mapping[:-1] > 0] // P)
    free_full = r_free.permutation(np.setdiff1d(np.arange(1, n_full // P + 1), used_full)).astype(np.int64)
    free_swa = r_free.permutation(np.setdiff1d(np.arange(1, n_swa // P + 1), used_swa)).astype(np.int64)
    rows = np.arange(1, B + 1)
    last = np.where(pre > 0, r2t[rows, np.maximum(pre - 1, 0)], -1).astype(np.int64)
    return AllocBatch(name, B, P, pre.astype(np.int32), seq.astype(np.int32), last, r2t, rows.astype(np.int32),
                      mapping, free_full, free_swa, n_full, n_swa)


def alloc_prefill_chunk(seed=SEED_BASE + 5, batch=256, chunk=2048) -> AllocBatch:
    """The fp8 decode batch (B = 256, lognormal lengths, P = 64) taking one more
    prefill chunk of 2048 positions per request."""
    pre = c5_lengths(seed, batch)
    return alloc_batch("alloc_chunk2048_B256", seed, pre, pre + chunk, 64)


def alloc_decode_step(seed=SEED_BASE + 5, batch=256) -> AllocBatch:
    """The fp8 decode batch's next decode step: one new position per request."""
    pre = c5_lengths(seed, batch)
    return alloc_batch("alloc_decode_B256", seed, pre, pre + 1, 64)


# ---------------------------------------------------------------------------
# Unified pool: virtual ids, a page table, and per-layer rows per live token
# (where the rows sit in the raw buffer is the layout under test, so it is
# not decided here)
# ---------------------------------------------------------------------------

@dataclass
class UnifiedBatch:
    name: str
    batch: int
    layers: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    page_size: int
    kv_dtype: str
    seq_lens: np.ndarray          # int32 (B,)
    req_to_token: np.ndarray      # int32 (B + 1, stride): virtual ids
    req_pool_idx: np.ndarray      # int32 (B,)
    v2p: np.ndarray               # int64 (virtual pages,): physical page, -1 tombstoned, v2p[0] = 0
    n_phys: int                   # physical pages of the sub-pool (page 0 included)
    live_tokens: np.ndarray       # int64: virtual ids whose page is live, ascending
    k_rows: Optional[np.ndarray]  # (layers, n_live, kv_heads, head_dim) storage bits, or None
    v_rows: Optional[np.ndarray]
    q: np.ndarray                 # (B, q_heads, head_dim) bf16 bits
    sinks: Optional[np.ndarray]
    new_k: np.ndarray             # (layers, B, kv_heads, head_dim) bf16 bits: the current token's K/V
    new_v: np.ndarray


def unified_batch(name, seed, seq_lens, layers, q_heads, kv_heads, window, page_size, kv_dtype="bf16", sinks=True,
                  live_margin=128, slack_pages=2, head_dim=128, with_rows=True) -> UnifiedBatch:
    """Decode requests over one unified SWA sub-pool of `layers` layers: virtual
    pages laid out like the two-pool decode workloads (the full-page
    permutation gives the virtual pages, the SWA-page permutation the physical
    pages of live pages; pages before seq - 1 - window - live_margin are
    tombstoned)."""
    r_len, r_full, r_swa, r_q, r_k, r_v, r_s, r_new = _streams(seed)
    seq = np.asarray(seq_lens, dtype=np.int64)
    B, P = len(seq), page_size
    n_virt = round_up(int(sum(round_up(int(t), P) for t in seq)) + slack_pages * P, P)
    live_from = np.maximum(seq - 1 - window - live_margin, 0)
    need = int(sum(round_up(int(t), P) - (int(lf) // P) * P for t, lf in zip(seq, live_from)))
    n_phys_tokens = round_up(need + slack_pages * P, P)
    r2t, mapping, _ = _layout(seq, P, n_virt, n_phys_tokens, live_from, r_full, r_swa)
    vp = np.arange(n_virt // P + 1)
    v2p = np.where(mapping[vp * P] > 0, mapping[vp * P] // P, -1).astype(np.int64)
    v2p[0] = 0
    live = np.nonzero(np.repeat(v2p > 0, P))[0].astype(np.int64)
    live = live[np.isin(live, r2t[1:][r2t[1:] > 0])]
    k_rows = v_rows = None
    if with_rows:
        k_rows = to_store(r_k.standard_normal((layers, live.size, kv_heads, head_dim), dtype=np.float32), kv_dtype)
        v_rows = to_store(r_v.standard_normal((layers, live.size, kv_heads, head_dim), dtype=np.float32), kv_dtype)
    q = to_store(r_q.standard_normal((B, q_heads, head_dim), dtype=np.float32), "bf16")
    s = r_s.standard_normal(q_heads).astype(np.float32) if sinks else None
    new_k = to_store(r_new.standard_normal((layers, B, kv_heads, head_dim), dtype=np.float32), "bf16")
    new_v = to_store(r_new.standard_normal((layers, B, kv_heads, head_dim), dtype=np.float32), "bf16")
    return UnifiedBatch(name, B, layers, q_heads, kv_heads, head_dim, window, P, kv_dtype, seq.astype(np.int32), r2t,
                        np.arange(1, B + 1, dtype=np.int32), v2p, n_phys_tokens // P + 1, live, k_rows, v_rows, q, s,
                        new_k, new_v)


def unified_c2_decode(seed=SEED_BASE + 2, layers=32) -> UnifiedBatch:
    """The batched SWA decode batch (B = 64, T ~ U[1024, 8192], W = 128, 64 q /
    8 kv heads, D = 128, bf16, P = 16, pages before the window tombstoned) over
    one unified sub-pool holding `layers` SWA layers; rows are left to the
    caller (the benchmark fills the buffer on the device)."""
    lens = np.random.default_rng(np.random.SeedSequence(seed).spawn(8)[0]).integers(1024, 8193, size=64)
    return unified_batch("unified_c2_B64_L%d" % layers, seed, lens, layers, 64, 8, 128, 16, live_margin=0,
                         with_rows=False)



# ---------------------------------------------------------------------------
# Per-request SWA ring: logical K/V of each request's live positions (which
# ring row holds a position is the layout under test, so it is not decided
# here)
# ---------------------------------------------------------------------------

@dataclass
class RingBatch:
    name: str
    batch: int
    q_heads: int
    kv_heads: int
    head_dim: int
    window: int
    request_slots: int            # request slots of the ring pool (slot 0 padding)
    seq_lens: np.ndarray          # int32 (B,)
    prefix_lens: np.ndarray       # int32 (B,): decode = seq - 1
    req_pool_idx: np.ndarray      # int32 (B,): distinct slots in 1 .. request_slots - 1
    live_lo: np.ndarray           # int64 (B,): first live position (the first query's first key)
    k_rows: List[np.ndarray]      # per request (prefix - live_lo, Hkv, D) bf16 bits: positions live_lo .. prefix-1
    v_rows: List[np.ndarray]
    q: np.ndarray                 # (sum of new positions, Hq, D) bf16 bits
    sinks: Optional[np.ndarray]
    new_k: np.ndarray             # (sum of new positions, Hkv, D) bf16 bits
    new_v: np.ndarray


def ring_batch(name, seed, prefix_lens, new_lens, q_heads, kv_heads, window, request_slots=None, sinks=True,
               head_dim=128) -> RingBatch:
    """Requests on seeded distinct request slots; each holds the K/V of the
    positions its next step reads from before its prefix (from the first new
    query's first key on) and brings new_lens new positions."""
    r_len, r_slot, _, r_q, r_k, r_v, r_s, r_new = _streams(seed)
    pre = np.asarray(prefix_lens, dtype=np.int64)
    new = np.asarray(new_lens, dtype=np.int64)
    B = len(pre)
    slots = request_slots or 2 * B + 2
    rows = (1 + r_slot.permutation(slots - 1)[:B]).astype(np.int32)
    lo = np.maximum(pre - window, 0) if window >= 0 else np.zeros(B, np.int64)
    k_rows = [to_store(r_k.standard_normal((int(p - l), kv_heads, head_dim), dtype=np.float32), "bf16")
              for p, l in zip(pre, lo)]
    v_rows = [to_store(r_v.standard_normal((int(p - l), kv_heads, head_dim), dtype=np.float32), "bf16")
              for p, l in zip(pre, lo)]
    total = int(new.sum())
    q = to_store(r_q.standard_normal((total, q_heads, head_dim), dtype=np.float32), "bf16")
    s = r_s.standard_normal(q_heads).astype(np.float32) if sinks else None
    new_k = to_store(r_new.standard_normal((total, kv_heads, head_dim), dtype=np.float32), "bf16")
    new_v = to_store(r_new.standard_normal((total, kv_heads, head_dim), dtype=np.float32), "bf16")
    return RingBatch(name, B, q_heads, kv_heads, head_dim, window, slots, (pre + new).astype(np.int32),
                     pre.astype(np.int32), rows, lo, k_rows, v_rows, q, s, new_k, new_v)
