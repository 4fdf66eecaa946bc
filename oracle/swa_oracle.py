"""Plain, slow CPU oracle of sliding-window attention (SWA) over a two-pool paged
KV cache, in float64 with numpy.

TEST INFRASTRUCTURE ONLY.  Only tests/, the smoke check and the CPU-baseline leg
of the benchmark may import it; the HIP library never does, and the two share
no code, headers, tables or helpers.

Sources (three web pages; every function names the passage it follows):
  [SWA]   zdszero.github.io/swa.html — SWA design note (sections: 问题 Problem,
          设计 Design, 抽象 Abstraction, 实现 Implementation, 双池与映射表
          Two pools and the mapping table, 显存怎么分 Memory split, 运行时
          Runtime, Attention backend).
  [POOLS] pinghaoyang.com.cn, "SGLang 源码完全拆解(十五): 内存池与显存管理"
          (sections: 一重映射 request-slot pool, 二重映射 KV storage pool,
          三重映射 page allocator, alloc_extend, 双池 + 映射表
          SWATokenToKVPoolAllocator, 谁在往页里写 who writes into the pages).

Readings taken where the pages are silent (each is listed in the design notes):
  * window: the configured W excludes the current token, so query i sees keys
    [max(0, i-W), i]; W = -1 means full attention ([SWA] 实现, per-layer
    sliding_window_size; FlashInfer path truncating to W+1 in Attention backend).
  * decode query position: i = seq_len - 1 (the current token's K/V is stored
    before attention).
  * sink: one extra logit sigma_h per q head in the softmax denominator, in the
    scaled-logit domain, with no value row ([SWA] 设计: weight "leaks" to the
    sink).  No sink is sigma = -inf.
  * softmax scale: 1/sqrt(D) unless the caller passes another.
  * GQA: q head h reads kv head floor(h / G), G = Hq / Hkv.
  * an in-window tombstone (mapping 0 on an SWA layer) is a contract violation
    and raises.
"""

from __future__ import annotations

import math

import numpy as np

from . import codecs


class OracleError(ValueError):
    """A contract violation detected by the oracle (bad index, tombstone...)."""


class NoSpaceError(OracleError):
    """The SWA pool cannot hold a single request (startup error on the pages)."""


# ---------------------------------------------------------------------------
# a1 — pool sizing.  [SWA] 显存怎么分 (--swa-full-tokens-ratio): with F and S
# the per-token, per-layer KV bytes of a full and of an SWA layer,
#   cell = F * L_full + r * S * L_swa,  N_full = floor(avail / cell),
#   N_swa = r * N_full,  both rounded down to a page;  N_swa <= W + P is a
# startup error.
# ---------------------------------------------------------------------------


def kv_bytes_per_token(kv_heads: int, head_dim: int, v_head_dim: int, dtype_size: int) -> int:
    """F or S of the cell formula: num_kv_heads * (head_dim + v_head_dim) * dtype_size."""
    return kv_heads * (head_dim + v_head_dim) * dtype_size


def pool_config(avail_bytes, ratio, page_size, window, n_full_layers, full_bytes_per_token,
                n_swa_layers, swa_bytes_per_token):
    """Return (cell_bytes, N_full, N_swa) for the two pools; raise NoSpaceError
    when N_swa <= W + P ([SWA] 显存怎么分)."""
    if page_size <= 0 or ratio < 0:
        raise OracleError("page_size must be positive and ratio non-negative")
    cell = full_bytes_per_token * n_full_layers + ratio * swa_bytes_per_token * n_swa_layers
    n_full = math.floor(avail_bytes / cell)
    n_full = (n_full // page_size) * page_size
    n_swa = math.floor(ratio * n_full)
    n_swa = (n_swa // page_size) * page_size
    if n_swa <= window + page_size:
        raise NoSpaceError(f"SWA pool of {n_swa} tokens cannot hold W + P = {window + page_size}")
    return cell, n_full, n_swa


# ---------------------------------------------------------------------------
# a2 — translate_loc.  [SWA] 双池与映射表 and Attention backend; [POOLS]
# 双池 + 映射表: the SWA index of a token is full_to_swa[full]; the table has
# size + page_size entries followed by one trailing -1, so -1 translates to -1;
# 0 means "no SWA slot" (tombstone / padding).
# ---------------------------------------------------------------------------


def translate_loc(full_loc, full_to_swa):
    """swa_loc[n] = full_to_swa[full_loc[n]], with -1 -> the trailing -1 entry.

    Any index outside [-1, len-2] is an error (the oracle does not clamp)."""
    m = np.asarray(full_to_swa, dtype=np.int64)
    x = np.asarray(full_loc, dtype=np.int64)
    if m.ndim != 1 or m.size < 2 or m[-1] != -1:
        raise OracleError("mapping table must end with the -1 sentinel")
    out = np.empty_like(x)
    for n, f in enumerate(x.tolist()):
        if f == -1:
            out[n] = m[m.size - 1]
        elif 0 <= f < m.size - 1:
            out[n] = m[f]
        else:
            raise OracleError(f"full loc {f} outside the mapping table")
    return out


# ---------------------------------------------------------------------------
# a3 — window gather.  [SWA] Attention backend: backends translate the window's
# full indices once per batch (FlashInfer keeps W+1 positions per request);
# [POOLS] 一重映射: req_to_token[row, pos] holds the full slot of each position.
# ---------------------------------------------------------------------------


def first_key(i: int, window: int, chunk: int = 0) -> int:
    """First key position query i sees: i - W for a sliding window (W >= 0),
    the start of i's chunk for chunked local attention (chunk C > 0: [SWA] 设计,
    Llama4's chunked local layers -- chunks of C positions from position 0, a
    query sees its own chunk up to itself), the larger of the two when both
    are given, and never below 0."""
    lo = 0
    if window >= 0:
        lo = max(lo, i - window)
    if chunk > 0:
        lo = max(lo, (i // chunk) * chunk)
    return lo


def window_range(seq_len: int, prefix_len: int, window: int, chunk: int = 0):
    """Positions [lo, hi] whose K/V the new queries of a request can see.

    The new queries are positions prefix_len .. seq_len-1; query i sees
    [first_key(i), i], so together they see [first_key(prefix_len), seq_len-1]
    (first_key never decreases with i).  Decode is prefix_len = seq_len - 1.
    W = -1 and chunk = 0 is full attention (lo = 0)."""
    hi = seq_len - 1
    lo = first_key(prefix_len, window, chunk)
    return lo, hi


def window_table(req_to_token, req_pool_idx, seq_lens, full_to_swa, window, prefix_lens=None, chunk=0):
    """Per request, the slots of positions window_range(...), concatenated.

    Returns (table int64, indptr int64 of length B+1).  With full_to_swa None
    the slots are the full-pool slots (full layers need no translation)."""
    r2t = np.asarray(req_to_token)
    rows = np.asarray(req_pool_idx, dtype=np.int64)
    lens = np.asarray(seq_lens, dtype=np.int64)
    b_count = lens.size
    pre = lens - 1 if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    table, indptr = [], [0]
    for b in range(b_count):
        lo, hi = window_range(int(lens[b]), int(pre[b]), window, chunk)
        for j in range(lo, hi + 1):
            full = int(r2t[rows[b], j])
            slot = full if full_to_swa is None else int(translate_loc([full], full_to_swa)[0])
            table.append(slot)
        indptr.append(len(table))
    return np.asarray(table, dtype=np.int64), np.asarray(indptr, dtype=np.int64)


# ---------------------------------------------------------------------------
# a4 — kv_store.  [SWA] Attention backend (KVWriteLoc: SWA layers receive an
# already translated swa_loc, the pool does not translate); [POOLS] 谁在往页里写
# and 二重映射 (per-layer k_buffer / v_buffer of shape (size + page, heads,
# dim); fp8 pools hold bytes).
# ---------------------------------------------------------------------------


def kv_store(pool_k, pool_v, loc, k_new, v_new, in_dtype: str, pool_dtype: str):
    """Return copies of the pools with row loc[n] set to enc(k_new[n]) / enc(v_new[n]).

    k_new / v_new hold storage bits of `in_dtype` with shape (n, Hkv, D); the
    pools hold storage bits of `pool_dtype` with shape (rows, Hkv, D).  Values
    are decoded exactly and re-encoded with the oracle codecs (a byte copy
    when the two dtypes agree).  Duplicate locs are a contract violation."""
    loc = np.asarray(loc, dtype=np.int64)
    if np.unique(loc).size != loc.size:
        raise OracleError("duplicate store locations")
    rows = pool_k.shape[0]
    if loc.size and (loc.min() < 0 or loc.max() >= rows):
        raise OracleError("store location outside the pool")
    out_k, out_v = pool_k.copy(), pool_v.copy()
    for n, slot in enumerate(loc.tolist()):
        out_k[slot] = codecs.encode_store(codecs.decode_store(k_new[n], in_dtype), pool_dtype)
        out_v[slot] = codecs.encode_store(codecs.decode_store(v_new[n], in_dtype), pool_dtype)
    return out_k, out_v


# ---------------------------------------------------------------------------
# a5 / a6 / a7 — attention.  [SWA] opening paragraph (each query attends only
# to the most recent window), 实现 (sliding_window_size excludes the current
# token, -1 = full) and 设计 (learnable per-head sink).
# ---------------------------------------------------------------------------


def attend(q, keys, values, sink, scale):
    """Output of one query head:

        s_j = scale * (q . k_j)
        m   = max(max_j s_j, sigma)
        o   = sum_j e^{s_j - m} v_j / (sum_j e^{s_j - m} + e^{sigma - m})

    sink None means sigma = -inf (plain softmax over the window)."""
    s = scale * (keys @ q)
    sigma = -math.inf if sink is None else float(sink)
    m = max(float(s.max()), sigma)
    w = np.exp(s - m)
    denom = w.sum() + (0.0 if sink is None else math.exp(sigma - m))
    return (w @ values) / denom


def _gather_kv(pool_k, pool_v, slots, pool_dtype, k_scale, v_scale):
    k = codecs.decode_store(pool_k[slots], pool_dtype) * k_scale
    v = codecs.decode_store(pool_v[slots], pool_dtype) * v_scale
    return k, v


def _slots_for(r2t_row, lo, hi, full_to_swa):
    full = np.asarray(r2t_row[lo:hi + 1], dtype=np.int64)
    if full_to_swa is None:
        return full
    slots = translate_loc(full, full_to_swa)
    if np.any(slots == 0):
        raise OracleError("in-window tombstone: a window position has no SWA slot")
    if np.any(slots < 0):
        raise OracleError("window position translated to the -1 sentinel")
    return slots


def attention(q, q_dtype, pool_k, pool_v, pool_dtype, req_to_token, req_pool_idx, seq_lens,
              full_to_swa, window, sinks=None, scale=None, prefix_lens=None, qo_indptr=None,
              k_scale=1.0, v_scale=1.0, only=None, chunk=0):
    """Windowed attention of the new queries of every request (decode or extend).

    q: storage bits (q_dtype) of shape (total_new, Hq, D); request b owns rows
    qo_indptr[b] .. qo_indptr[b+1]-1, holding positions prefix_lens[b] .. seq_lens[b]-1.
    Decode is prefix_lens = seq_lens - 1 with one row per request (the defaults).
    pool_k / pool_v: storage bits of shape (rows, Hkv, D).  full_to_swa None means
    the pool is the full pool.  Returns float64 (total_new, Hq, D), unrounded.

    `only`, if given, is a list of (row, head) pairs to compute; other entries
    are left NaN (for sampled checks at full size)."""
    qf = codecs.decode_store(q, q_dtype)
    total_new, hq, d = qf.shape
    hkv = pool_k.shape[1]
    if hq % hkv:
        raise OracleError("q heads must be a multiple of kv heads")
    group = hq // hkv
    lens = np.asarray(seq_lens, dtype=np.int64)
    b_count = lens.size
    pre = lens - 1 if prefix_lens is None else np.asarray(prefix_lens, dtype=np.int64)
    indptr = np.arange(b_count + 1) if qo_indptr is None else np.asarray(qo_indptr, dtype=np.int64)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    r2t = np.asarray(req_to_token)
    rows = np.asarray(req_pool_idx, dtype=np.int64)
    out = np.full((total_new, hq, d), np.nan)
    wanted = None if only is None else {}
    if only is not None:
        for r, h in only:
            wanted.setdefault(int(r), []).append(int(h))
    for b in range(b_count):
        if indptr[b + 1] - indptr[b] != lens[b] - pre[b]:
            raise OracleError("qo_indptr disagrees with seq_lens - prefix_lens")
        for t in range(int(indptr[b + 1] - indptr[b])):
            row = int(indptr[b] + t)
            if wanted is not None and row not in wanted:
                continue
            i = int(pre[b]) + t
            lo = first_key(i, window, chunk)
            slots = _slots_for(r2t[rows[b]], lo, i, full_to_swa)
            k, v = _gather_kv(pool_k, pool_v, slots, pool_dtype, k_scale, v_scale)
            heads = range(hq) if wanted is None else wanted[row]
            for h in heads:
                g = h // group
                sink = None if sinks is None else sinks[h]
                out[row, h] = attend(qf[row, h], k[:, g, :], v[:, g, :], sink, scale)
    return out


def decode(q, q_dtype, pool_k, pool_v, pool_dtype, req_to_token, req_pool_idx, seq_lens,
           full_to_swa, window, sinks=None, scale=None, k_scale=1.0, v_scale=1.0, only=None, chunk=0):
    """Decode: one query per request at position seq_len-1 (see attention)."""
    return attention(q, q_dtype, pool_k, pool_v, pool_dtype, req_to_token, req_pool_idx,
                     seq_lens, full_to_swa, window, sinks, scale, None, None, k_scale, v_scale, only, chunk)


def extend(q, q_dtype, qo_indptr, prefix_lens, pool_k, pool_v, pool_dtype, req_to_token,
           req_pool_idx, seq_lens, full_to_swa, window, sinks=None, scale=None,
           k_scale=1.0, v_scale=1.0, only=None, chunk=0):
    """Extend / chunked prefill: queries prefix_len .. seq_len-1 per request,
    each over [first_key(i), i], against a pool that already holds the chunk's
    K/V (see attention)."""
    return attention(q, q_dtype, pool_k, pool_v, pool_dtype, req_to_token, req_pool_idx,
                     seq_lens, full_to_swa, window, sinks, scale, prefix_lens, qo_indptr,
                     k_scale, v_scale, only, chunk)


# ---------------------------------------------------------------------------
# Per-request SWA ring.  [POOLS] SWATokenToKVPoolAllocator ("为什么滑窗可以
# 按请求记账"): with a ring, each request slot owns a fixed SWA capacity of the
# ring size rounded up to a page, total capacity = request slots x that cost,
# and the paged SWA indices go unused.  Reading: slot r owns rows
# [r*R, (r+1)*R) and position j lives at row r*R + j mod R, so a request's
# positions overwrite their own ring and no mapping or eviction is needed; it
# is valid while the positions a step reads or writes span at most R.
# ---------------------------------------------------------------------------


def ring_rows(ring_size: int, page_size: int) -> int:
    """R: the ring size rounded up to a whole page (_swa_ring_cost)."""
    return -(-ring_size // page_size) * page_size


def ring_capacity(request_slots: int, ring_size: int, page_size: int) -> int:
    """The SWA pool's capacity in ring mode: every request slot's ring."""
    return request_slots * ring_rows(ring_size, page_size)


def ring_slot(row: int, pos: int, R: int) -> int:
    return row * R + pos % R


def ring_req_to_token(n_rows: int, stride: int, R: int):
    """The table of ring slots: entry [r, j] = ring_slot(r, j, R), int64.
    Attention over a ring is attention with these slots read directly
    (full_to_swa None)."""
    r = np.arange(n_rows, dtype=np.int64)[:, None]
    j = np.arange(stride, dtype=np.int64)[None, :]
    return r * R + j % R


# ---------------------------------------------------------------------------
# f1 — SWA eviction.  [SWA] 运行时 (free_swa_out_of_window_slots): per request,
# the SWA KV of positions that left the window is returned to the SWA pool:
# lower bound the larger of the request's evicted length and its protected
# (radix-managed) prefix, upper bound pre_len - W (chunk cache) or
# pre_len - max(W, page) (radix cache), aligned down to a page; in decode the
# release waits until at least `interval` (128 by default) tokens have left the
# window.  [SWA] 双池与映射表: free_swa releases only mapping values > 0 and then
# zeroes them, so a repeated release frees nothing twice.
# ---------------------------------------------------------------------------

RADIX = 1  # mode: radix cache (upper bound pre_len - max(W, P)); 0 = chunk cache


def evict_range(pre_len, evicted, protected, window, page_size, mode, interval):
    """(lo, hi) of the positions to release for one request; hi <= lo means none."""
    bound = pre_len - (max(window, page_size) if mode == RADIX else window)
    hi = (bound // page_size) * page_size if bound > 0 else 0
    lo = max(evicted, protected)
    if interval > 0 and hi - evicted < interval:
        return lo, lo
    return lo, hi


def evict(req_to_token, req_pool_idx, full_to_swa, pre_lens, evicted_lens, window, page_size, mode=0,
          interval=0, protected_lens=None):
    """Release the out-of-window SWA slots of every request.

    Returns (mapping, evicted_lens, freed_pages): a new mapping with the released
    entries set to 0, the advanced evicted lengths (a request with nothing to
    release keeps its value), and the released SWA pages in request order, then
    position order.  A page is reported at the first released position of the
    range and at every released position that starts a page (slot // page)."""
    r2t = np.asarray(req_to_token)
    m = np.array(full_to_swa, dtype=np.int64, copy=True)
    ev = np.array(evicted_lens, dtype=np.int64, copy=True)
    pages = []
    for b in range(len(pre_lens)):
        prot = 0 if protected_lens is None else int(protected_lens[b])
        lo, hi = evict_range(int(pre_lens[b]), int(ev[b]), prot, window, page_size, mode, interval)
        if hi <= lo:
            continue
        row = int(req_pool_idx[b])
        for j in range(lo, hi):
            full = int(r2t[row, j])
            slot = int(m[full])
            if slot > 0:
                if j == lo or j % page_size == 0:
                    pages.append(slot // page_size)
                m[full] = 0
        ev[b] = hi
    return m, ev, np.asarray(pages, dtype=np.int64)


# ---------------------------------------------------------------------------
# Paired allocation.  [POOLS] 三重映射 (a paged allocator hands out pages from
# the head of its free list; page 0 is never free), alloc_extend (per request:
# where its outputs start and where its new pages start in the free list, then
# three parts: the rest of the half-full page from last_loc + 1, whole new
# pages, the tail page), alloc_decode (one token per request), 扩容与不足
# (the optimistic bound extend_tokens // P + bs + 1, else the exact count;
# not enough pages -> nothing is allocated), and 双池 + 映射表 together with
# [SWA] 双池与映射表 (both allocators allocate the same count, the SWA side's
# last_loc is the mapping of the full one -- the trailing -1 turns a -1 into
# -1 -- and the mapping is written afterwards).
# ---------------------------------------------------------------------------


def _ceil_div(a: int, b: int) -> int:
    return -(-a // b)


def pages_needed(pre_lens, seq_lens, page_size) -> int:
    """Exact number of new pages: sum over requests of ceil(seq/P) - ceil(pre/P)
    ([POOLS] alloc_extend, the page-count formula)."""
    return int(sum(_ceil_div(int(s), page_size) - _ceil_div(int(p), page_size)
                   for p, s in zip(pre_lens, seq_lens)))


def pages_bound(extend_num_tokens, batch, page_size) -> int:
    """The optimistic upper bound of [POOLS] 扩容与不足."""
    return int(extend_num_tokens) // page_size + int(batch) + 1


def alloc_extend(pre_lens, seq_lens, last_loc, free_pages, page_size):
    """One pool's allocation of the slots of positions [pre_len, seq_len) of
    every request.  Returns (out, pages_taken) with out in request order, or
    None when the free list is too short.  Follows [POOLS] alloc_extend."""
    P = page_size
    free_pages = np.asarray(free_pages, dtype=np.int64)
    if pages_needed(pre_lens, seq_lens, P) > free_pages.size:
        return None
    out = []
    new_page_start = 0  # running prefix sum of the earlier requests' new pages
    for pre, seq, last in zip(pre_lens, seq_lens, last_loc):
        pre, seq, last = int(pre), int(seq), int(last)
        own_pages = _ceil_div(seq, P) - _ceil_div(pre, P)
        # part 1: the rest of the page the prefix ends in, continuing from last_loc
        n1 = min(seq, _ceil_div(pre, P) * P) - pre
        out.extend(last + 1 + k for k in range(n1))
        if pre + n1 < seq:
            # part 2: whole new pages
            n2 = (seq // P) * P - _ceil_div(pre, P) * P
            for off in range(n2):
                page = int(free_pages[new_page_start + off // P])
                out.append(page * P + off % P)
            # part 3: the tail, at the start of the last new page
            n3 = seq - (seq // P) * P
            if n3 > 0:
                page = int(free_pages[new_page_start + own_pages - 1])
                out.extend(page * P + k for k in range(n3))
        new_page_start += own_pages
    return np.asarray(out, dtype=np.int64), new_page_start


def alloc_decode(seq_lens, last_loc, free_pages, page_size):
    """One new token per request (pre_len = seq_len - 1): last_loc + 1 while it
    stays in its page, else the start of the next free page.  Returns
    (out, pages_taken) or None.  Follows [POOLS] alloc_decode."""
    P = page_size
    free_pages = np.asarray(free_pages, dtype=np.int64)
    pre_lens = [int(s) - 1 for s in seq_lens]
    if pages_needed(pre_lens, seq_lens, P) > free_pages.size:
        return None
    out = []
    new_page_start = 0
    for seq, last in zip(seq_lens, last_loc):
        seq, pre = int(seq), int(seq) - 1
        own = _ceil_div(seq, P) - _ceil_div(pre, P)
        if own == 0:
            out.append(int(last) + 1)
        else:
            out.append(int(free_pages[new_page_start]) * P)
        new_page_start += own
    return np.asarray(out, dtype=np.int64), new_page_start


def alloc_paired(pre_lens, seq_lens, last_loc, full_free, swa_free, full_to_swa, page_size, decode=False):
    """SWATokenToKVPoolAllocator: the same allocation on the full and the SWA
    pool, the SWA side continuing from full_to_swa[last_loc] (index -1 reads the
    trailing -1), then full_to_swa[full_out] = swa_out.  Returns (full_out,
    swa_out, mapping, pages_taken) or None if either free list is too short.
    With swa_free None (one pool) only the full allocation is made."""
    m = np.array(full_to_swa, dtype=np.int64, copy=True) if full_to_swa is not None else None
    if decode:
        full = alloc_decode(seq_lens, last_loc, full_free, page_size)
    else:
        full = alloc_extend(pre_lens, seq_lens, last_loc, full_free, page_size)
    if full is None:
        return None
    if swa_free is None:
        return full[0], None, m, full[1]
    swa_last = [int(m[int(x)]) for x in last_loc]  # Python's m[-1] is the sentinel
    if decode:
        swa = alloc_decode(seq_lens, swa_last, swa_free, page_size)
    else:
        swa = alloc_extend(pre_lens, seq_lens, swa_last, swa_free, page_size)
    if swa is None:
        return None
    m[full[0]] = swa[0]
    return full[0], swa[0], m, full[1]


# ---------------------------------------------------------------------------
# Unified pool.  [PR] (prhub.com.cn digest of sglang pull request 34602),
# 功能与动机 and 实现拆解: one raw byte buffer stores every layer's K/V in
# page-major envelopes [L0_K*ps | L0_V*ps | L1_K*ps | ...], i.e. 2L equally
# wide row blocks per page; layer l's K is block 2l and its V block 2l + 1.
# Per-layer dense views start at their block and address rows by the
# kernel-facing id kernel_id(t) = v2p[t // ps] * (ps * 2L) + t % ps, a
# tombstoned page (-1) clamped to 0, the page-0 sink; the last view reaches
# (2L - 1) * ps rows past the last envelope, so one envelope of tail padding
# follows the buffer; kernel-facing rows must stay below 2^31.
# ---------------------------------------------------------------------------


def unified_geometry(layer_num, kv_heads, head_dim, itemsize, page_size, num_pages):
    """Sizes of one sub-pool: row bytes, row blocks per page, envelope bytes,
    kernel-facing rows, envelope bytes in all, and the tail pad."""
    row_bytes = kv_heads * head_dim * itemsize
    blocks = 2 * layer_num
    page_bytes = page_size * blocks * row_bytes
    return dict(row_bytes=row_bytes, blocks=blocks, page_bytes=page_bytes, n_rows=num_pages * blocks * page_size,
                total_bytes=num_pages * page_bytes, tail_pad=page_bytes)


def envelope_offset(anchor, phys_page, layer, kv, offset, layer_num, row_bytes, page_size):
    """Byte offset of one row in the page-major envelope: page phys_page, block
    2 * layer + kv (kv 0 = K, 1 = V), in-page offset `offset`."""
    return anchor + ((phys_page * 2 * layer_num + 2 * layer + kv) * page_size + offset) * row_bytes


def unified_view_base(anchor, layer, kv, row_bytes, page_size):
    """Start byte of layer `layer`'s K (kv 0) or V (kv 1) dense view: its block
    in page 0's envelope."""
    return anchor + (2 * layer + kv) * page_size * row_bytes


def unified_kernel_ids(virt, v2p, page_size, multiplier):
    """translate_kv_loc_for_kernel: kernel_id = v2p[t // ps] * (ps * multiplier)
    + t % ps, then clamped at 0.  Virtual ids must be >= 0 and inside the page
    table."""
    virt = np.asarray(virt, dtype=np.int64)
    v2p = np.asarray(v2p, dtype=np.int64)
    pages = virt // page_size
    if virt.size and (virt.min() < 0 or pages.max() >= v2p.size):
        raise OracleError("virtual id outside the page table")
    ids = v2p[pages] * (page_size * multiplier) + virt % page_size
    return np.maximum(ids, 0)


def unified_mapping(v2p, page_size, multiplier):
    """The per-virtual-token kernel ids as a mapping table (tombstones 0, a
    trailing -1), so that window attention over a unified view is the same
    computation as over a two-pool SWA layer."""
    n_virt = len(v2p) * page_size
    m = unified_kernel_ids(np.arange(n_virt), v2p, page_size, multiplier)
    return np.concatenate([m, [-1]]).astype(np.int64)


def unified_views(raw, anchor, layer_num, kv_heads, head_dim, store_dtype, page_size, num_pages):
    """The per-layer dense views, built as numpy strided views over the raw
    byte buffer (the buffer must hold the tail pad).  store_dtype: numpy dtype
    of the stored elements (np.uint16 for bf16 bits, np.uint8 for e4m3,
    np.float32).  Returns ([K_0, ...], [V_0, ...]), each (n_rows, H, D)."""
    itemsize = np.dtype(store_dtype).itemsize
    g = unified_geometry(layer_num, kv_heads, head_dim, itemsize, page_size, num_pages)
    ks, vs = [], []
    for layer in range(layer_num):
        for kv, out in ((0, ks), (1, vs)):
            base = unified_view_base(anchor, layer, kv, g["row_bytes"], page_size)
            end = base + g["n_rows"] * g["row_bytes"]
            if end > raw.size:
                raise OracleError(f"view of layer {layer} ends at byte {end}; the buffer holds {raw.size}")
            out.append(np.lib.stride_tricks.as_strided(
                raw[base:].view(store_dtype), shape=(g["n_rows"], kv_heads, head_dim),
                strides=(g["row_bytes"], head_dim * itemsize, itemsize), writeable=False))
    return ks, vs


# ---------------------------------------------------------------------------
# Index-data contracts, counted rather than raised.  [SWA] 双池与映射表 and
# 运行时: a live window never holds a tombstone (eviction frees only positions
# that left the window) and the mapping ends in the -1 sentinel that a -1 loc
# reads; [POOLS] 一重映射 and 二重映射: indices stay inside their tables and
# page 0 is the shared sink of padded writes; 释放: a slot is handed out once.
# ---------------------------------------------------------------------------

VALIDATE_FIELDS = ("bad_requests", "positions", "full_out_of_range", "tombstones", "sentinels",
                   "slot_out_of_range", "store_locs", "store_out_of_range", "store_duplicates", "qo_bad")


def validate(req_to_token, req_pool_idx, seq_lens, full_to_swa, window, pool_rows, page_size,
             prefix_lens=None, store_loc=None, qo_indptr=None, total_q=0):
    """Counts of violations in a batch's index data.

    A request is bad when its req_to_token row, its length or its prefix lies
    outside its table; its window is then skipped.  Each window position (the
    positions window_range gives) is classified once: a full slot outside the
    mapping (with a mapping), a tombstone (slot 0), the sentinel (slot -1) or
    another slot outside [0, pool_rows).  Store locations: outside
    [0, pool_rows), or a repeat of a location outside page 0.  Query rows of
    an extend (qo_indptr given): a request whose rows qo_indptr[b] ..
    qo_indptr[b+1]-1 are not in order inside [0, total_q], or, when it is not
    bad and prefix_lens is given, are not its seq - prefix new positions."""
    r2t = np.asarray(req_to_token)
    n_rows, stride = r2t.shape
    c = dict.fromkeys(VALIDATE_FIELDS, 0)
    for b in range(len(seq_lens)):
        row, n = int(req_pool_idx[b]), int(seq_lens[b])
        pre = n - 1 if prefix_lens is None else int(prefix_lens[b])
        bad = not (0 <= row < n_rows) or not (0 <= n <= stride) or (prefix_lens is not None and not 0 <= pre <= n)
        if qo_indptr is not None:
            q0, q1 = int(qo_indptr[b]), int(qo_indptr[b + 1])
            if not 0 <= q0 <= q1 <= total_q or (not bad and prefix_lens is not None and q1 - q0 != n - pre):
                c["qo_bad"] += 1
        if bad:
            c["bad_requests"] += 1
            continue
        if n == 0:
            continue
        lo = 0 if window < 0 else max(0, pre - window)
        for j in range(lo, n):
            c["positions"] += 1
            full = int(r2t[row, j])
            if full_to_swa is not None:
                if not -1 <= full < len(full_to_swa) - 1:
                    c["full_out_of_range"] += 1
                    continue
                slot = int(full_to_swa[full])  # full = -1 reads the trailing sentinel entry
                if slot == 0:
                    c["tombstones"] += 1
                elif slot == -1:
                    c["sentinels"] += 1
                elif not 0 <= slot < pool_rows:
                    c["slot_out_of_range"] += 1
            elif full == 0:
                c["tombstones"] += 1
            elif not 0 <= full < pool_rows:
                c["slot_out_of_range"] += 1
    if store_loc is not None:
        seen = set()
        for x in (int(v) for v in store_loc):
            c["store_locs"] += 1
            if not 0 <= x < pool_rows:
                c["store_out_of_range"] += 1
            elif x >= page_size:
                if x in seen:
                    c["store_duplicates"] += 1
                seen.add(x)
    return c


# ---------------------------------------------------------------------------
# Cost model.  [SWA] 问题: causal full attention scores about T^2/2 pairs, SWA
# a fixed window per query; the ratio is about 2W/T.
# ---------------------------------------------------------------------------


def scored_pairs(seq_len: int, window: int) -> int:
    """Number of (query, key) pairs the oracle scores for one request of length
    T when every position is a query (prefill), counted by walking the windows."""
    total = 0
    for i in range(seq_len):
        lo = 0 if window < 0 else max(0, i - window)
        total += i - lo + 1
    return total
