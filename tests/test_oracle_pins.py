"""Pins of the CPU oracle against facts fixed by the pages and by mathematics.

Every check here is independent of the oracle's own code path: textbook matrix
attention, pure-Python loops, closed forms, library casts, page-level rebuilds
of the index tables, and figures printed on the pages (tests/golden).
"""

import json
import math
import os

import numpy as np
import pytest
import scipy.special
import torch

from oracle import codecs
from oracle import swa_oracle as O
from sliding_window_attention_swa_amd import workloads as WL

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "pages_figures.json")


def golden():
    with open(GOLDEN) as f:
        return json.load(f)


# ---------------------------------------------------------------------------
# codecs against torch's casts (library routines)
# ---------------------------------------------------------------------------

ALL_BF16 = np.arange(65536, dtype=np.uint32).astype(np.uint16)


def test_bf16_decode_matches_torch_on_every_pattern():
    ours = codecs.bf16_bits_to_f64(ALL_BF16)
    ref = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()


def test_bf16_encode_matches_torch():
    rng = np.random.default_rng(1)
    x = np.concatenate([
        rng.standard_normal(200000).astype(np.float32),
        (rng.standard_normal(20000) * 1e-38).astype(np.float32),  # subnormal range
        (rng.standard_normal(20000) * 1e30).astype(np.float32),
        # exact ties: bf16 values plus half an ulp (odd and even mantissas)
        (codecs.bf16_bits_to_f64(np.arange(0x3F80, 0x3FA0, dtype=np.uint16)) * (1 + 2.0 ** -8)).astype(np.float32),
        np.array([0.0, -0.0, 1.0, -1.0, 3.0e38, -3.0e38], dtype=np.float32),
    ])
    ours = codecs.f64_to_bf16_bits(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_e4m3_decode_matches_torch_on_every_code():
    codes = np.arange(256, dtype=np.uint8)
    ours = codecs.e4m3_to_f64(codes)
    ref = torch.from_numpy(codes).view(torch.float8_e4m3fn).to(torch.float64).numpy()
    same = (ours == ref) | (np.isnan(ours) & np.isnan(ref))
    assert same.all()
    assert codecs.e4m3_to_f64(np.array([0x7E]))[0] == 448.0


def test_e4m3_encode_matches_torch_on_every_bf16_input():
    vals = codecs.bf16_bits_to_f64(ALL_BF16)
    ours = codecs.f64_to_e4m3(vals)
    ref = torch.from_numpy(ALL_BF16.view(np.int16)).view(torch.bfloat16).to(torch.float8_e4m3fn) \
        .view(torch.uint8).numpy()
    finite_in_range = np.isfinite(vals) & (np.abs(vals) <= 464.0)
    assert np.array_equal(ours[finite_in_range], ref[finite_in_range])
    # reading: saturate-to-finite beyond the largest finite value, NaN -> 0x7F
    big = np.isfinite(vals) & (np.abs(vals) > 448.0) | np.isinf(vals)
    assert np.all(codecs.e4m3_to_f64(ours[big]) == np.sign(vals[big]) * 448.0)
    assert np.all(ours[np.isnan(vals)] == 0x7F)


def test_e4m3_encode_fp32_inputs_match_torch():
    rng = np.random.default_rng(2)
    x = np.concatenate([rng.standard_normal(100000), rng.standard_normal(20000) * 1e-3,
                        rng.uniform(-460, 460, 20000)]).astype(np.float32)
    ours = codecs.f64_to_e4m3(x.astype(np.float64))
    ref = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, ref)


# ---------------------------------------------------------------------------
# pool sizing: the MiMo-V2-Flash worked example printed on the SWA note
# ---------------------------------------------------------------------------


def test_pool_config_reproduces_mimo_example():
    g = golden()["mimo_pool_split"]
    F = 1000  # bytes per token per full layer; S = 2F
    S = int(F * g["swa_bytes_over_full_bytes"])
    avail = 10 ** 12
    cells = {}
    for case in g["cases"]:
        cell, n_full, n_swa = O.pool_config(avail, case["ratio"], 1, 128, g["layers_full"], F,
                                            g["layers_swa"], S)
        assert round(cell / F, 1) == case["cell_over_F"]
        cells[case["ratio"]] = (cell, n_full, n_swa)
        if "swa_share_of_kv_memory_approx" in case:
            share = n_swa * S * g["layers_swa"] / (n_swa * S * g["layers_swa"] + n_full * F * g["layers_full"])
            assert round(share, 2) == case["swa_share_of_kv_memory_approx"]
    gain = cells[0.05][1] / cells[0.8][1]
    assert round(gain, 1) == g["cases"][1]["full_capacity_gain_vs_ratio_0.8_approx"]


def test_pool_config_page_rounding_and_nospace():
    # rounding down to a page on both pools
    cell, n_full, n_swa = O.pool_config(10 ** 9, 0.1, 64, 128, 9, 2048, 39, 4096)
    assert n_full % 64 == 0 and n_swa % 64 == 0
    assert n_full <= 10 ** 9 / cell < n_full + 64
    # the long-context mixed configuration: 32 requests x 32K tokens fill the full pool
    F = O.kv_bytes_per_token(4, 128, 128, 2)
    S = O.kv_bytes_per_token(8, 128, 128, 2)
    assert (F, S) == (2048, 4096)
    cell = F * 9 + 0.1 * S * 39
    _, n_full, n_swa = O.pool_config(math.ceil(cell * 1048576), 0.1, 64, 128, 9, F, 39, S)
    assert n_full == 1048576 and n_swa == 104832
    # startup error when the SWA pool cannot hold W + P tokens
    with pytest.raises(O.NoSpaceError):
        O.pool_config(192 * 4096 * 10, 0.01, 64, 128, 0, 0, 10, 4096)


# ---------------------------------------------------------------------------
# index translation against page-level rebuilds (slot = page * P + offset)
# ---------------------------------------------------------------------------


def test_page_math_examples():
    """The page maths the Pools article prints (slot = page x size + offset,
    page = slot // size), through the oracle's allocator: a request that starts
    a fresh page gets, at in-page offset k, the slot page x size + k of the page
    its free list hands out."""
    for ex in golden()["page_math"]["examples"]:
        P, page, off = ex["page_size"], ex["page"], ex["offset"]
        out, taken = O.alloc_extend(np.array([0]), np.array([off + 1]), np.array([-1]), np.array([page]), P)
        assert taken == 1 and int(out[off]) == ex["slot"]
        assert int(out[off]) // P == page


def make_two_pool(rng, seq_lens, P, window, margin, n_full_pages=None, n_swa_pages=None):
    """A page-consistent two-pool cache described at page level.

    Returns the token-level tables plus the page-level truth used to rebuild
    expected slots: full_pages[b][p] and swa_pages[b][p] (0 when tombstoned)."""
    B = len(seq_lens)
    need = [-(-t // P) for t in seq_lens]
    n_full_pages = n_full_pages or sum(need) + 3
    n_swa_pages = n_swa_pages or sum(need) + 3
    fperm = rng.permutation(np.arange(1, n_full_pages + 1))
    sperm = rng.permutation(np.arange(1, n_swa_pages + 1))
    stride = max(seq_lens) + 5
    r2t = np.zeros((B + 1, stride), dtype=np.int32)
    mapping = np.zeros((n_full_pages + 1) * P + 1, dtype=np.int64)
    mapping[-1] = -1
    full_pages, swa_pages = [], []
    fi = si = 0
    for b, t in enumerate(seq_lens):
        fp = fperm[fi:fi + need[b]]
        fi += need[b]
        keep_from = max(0, (t - 1 - window - margin)) // P if window >= 0 else 0
        sp = np.zeros(need[b], dtype=np.int64)
        for p in range(keep_from, need[b]):
            sp[p] = sperm[si]
            si += 1
        full_pages.append(fp)
        swa_pages.append(sp)
        for j in range(t):
            p, k = divmod(j, P)
            r2t[b + 1, j] = fp[p] * P + k
            mapping[fp[p] * P + k] = 0 if sp[p] == 0 else sp[p] * P + k
    return r2t, np.arange(1, B + 1, dtype=np.int32), np.asarray(seq_lens, np.int32), mapping, full_pages, swa_pages


def test_translate_loc_invariants_and_page_rebuild():
    rng = np.random.default_rng(3)
    P = 4
    r2t, rows, lens, mapping, fpages, spages = make_two_pool(rng, [37, 9, 50], P, 6, 2)
    assert mapping[-1] == -1
    out = O.translate_loc(np.array([-1, 0, 0, -1]), mapping)
    assert out.tolist() == [-1, 0, 0, -1]
    for b, t in enumerate(lens):
        full = r2t[b + 1, :t]
        got = O.translate_loc(full, mapping)
        want = [0 if spages[b][j // P] == 0 else spages[b][j // P] * P + j % P for j in range(t)]
        assert got.tolist() == want
    with pytest.raises(O.OracleError):
        O.translate_loc(np.array([mapping.size - 1]), mapping)
    with pytest.raises(O.OracleError):
        O.translate_loc(np.array([-2]), mapping)


@pytest.mark.parametrize("window", [0, 3, 6, 100, -1])
def test_window_table_page_rebuild(window):
    rng = np.random.default_rng(4)
    P = 4
    lens = [37, 1, 9, 50]
    r2t, rows, lens_a, mapping, fpages, spages = make_two_pool(rng, lens, P, max(window, 0), 3)
    for use_map in (True, False):
        if window < 0 and use_map:
            continue
        table, indptr = O.window_table(r2t, rows, lens_a, mapping if use_map else None, window)
        assert indptr[0] == 0 and indptr.size == len(lens) + 1
        for b, t in enumerate(lens):
            i = t - 1
            lo = 0 if window < 0 else max(0, i - window)
            pages = spages[b] if use_map else fpages[b]
            want = [pages[j // P] * P + j % P for j in range(lo, i + 1)]
            assert table[indptr[b]:indptr[b + 1]].tolist() == want
            assert indptr[b + 1] - indptr[b] == (t if window < 0 else min(t, window + 1))


def test_window_table_extend_ranges():
    rng = np.random.default_rng(5)
    P = 8
    lens = [40, 24]
    pre = [30, 0]
    r2t, rows, lens_a, mapping, fpages, spages = make_two_pool(rng, lens, P, 5, 1)
    table, indptr = O.window_table(r2t, rows, lens_a, mapping, 5, prefix_lens=np.array(pre))
    assert (indptr[1] - indptr[0]) == 40 - 25
    assert (indptr[2] - indptr[1]) == 24


# ---------------------------------------------------------------------------
# kv_store: round trip and untouched rows
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("in_dtype,pool_dtype", [("bf16", "bf16"), ("f32", "f32"), ("bf16", "e4m3"),
                                                 ("f32", "e4m3"), ("f32", "bf16")])
def test_kv_store_round_trip(in_dtype, pool_dtype):
    rng = np.random.default_rng(6)
    rows, H, D, n = 40, 2, 8, 7
    x = rng.standard_normal((n, H, D)) * 3
    k_new = codecs.encode_store(x, in_dtype)
    v_new = codecs.encode_store(-x, in_dtype)
    empty = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[pool_dtype]
    pool_k = np.full((rows, H, D), 0x55, dtype=empty)
    pool_v = np.full((rows, H, D), 0x66, dtype=empty)
    loc = rng.choice(np.arange(1, rows), n, replace=False)
    nk, nv = O.kv_store(pool_k, pool_v, loc, k_new, v_new, in_dtype, pool_dtype)
    other = np.setdiff1d(np.arange(rows), loc)
    assert np.array_equal(nk[other], pool_k[other]) and np.array_equal(nv[other], pool_v[other])
    src = codecs.decode_store(k_new, in_dtype)
    got = codecs.decode_store(nk[loc], pool_dtype)
    if in_dtype == pool_dtype:
        assert np.array_equal(nk[loc].view(np.uint8), k_new.view(np.uint8))
        assert np.array_equal(nv[loc].view(np.uint8), v_new.view(np.uint8))
    else:
        # the stored value is a nearest representable value of the target format
        table = codecs.E4M3_VALUES[np.isfinite(codecs.E4M3_VALUES)] if pool_dtype == "e4m3" else None
        if table is not None:
            best = np.min(np.abs(src[..., None] - table), axis=-1)
            assert np.allclose(np.abs(src - got), best, rtol=0, atol=0)
        else:
            assert np.all(np.abs(src - got) <= np.abs(src) * 2.0 ** -8)
    with pytest.raises(O.OracleError):
        O.kv_store(pool_k, pool_v, np.array([3, 3]), k_new[:2], v_new[:2], in_dtype, pool_dtype)


# ---------------------------------------------------------------------------
# attention
# ---------------------------------------------------------------------------


def dense_case(rng, T, Hq, Hkv, D, window, P=1, margin=0, qdt="f32", kvdt="f32", sinks=True, evict=False):
    """One request whose every position is a query (prefix 0), on a shuffled
    two-pool cache; returns arguments for O.extend plus the dense logical K/V.
    With evict=True, pages before the last window (+ margin) are tombstoned,
    which only a decode of the last position may read around."""
    keep = max(window, 0) if evict else T
    r2t, rows, lens, mapping, fpages, spages = make_two_pool(rng, [T], P, keep, margin)
    n_rows = mapping.size
    q = codecs.encode_store(rng.standard_normal((T, Hq, D)), qdt)
    kd = codecs.encode_store(rng.standard_normal((T, Hkv, D)), kvdt)
    vd = codecs.encode_store(rng.standard_normal((T, Hkv, D)), kvdt)
    empty = {"f32": np.float32, "bf16": np.uint16, "e4m3": np.uint8}[kvdt]
    nan_bits = {"f32": np.float32(np.nan), "bf16": np.uint16(0x7FC0), "e4m3": np.uint8(0x7F)}[kvdt]
    pool_k = np.full((n_rows, Hkv, D), nan_bits, dtype=empty)
    pool_v = np.full((n_rows, Hkv, D), nan_bits, dtype=empty)
    use_map = window >= 0
    for j in range(T):
        full = r2t[1, j]
        slot = mapping[full] if use_map else full
        if slot > 0:
            pool_k[slot] = kd[j]
            pool_v[slot] = vd[j]
    s = rng.standard_normal(Hq) if sinks else None
    args = dict(q=q, q_dtype=qdt, qo_indptr=np.array([0, T]), prefix_lens=np.array([0]), pool_k=pool_k,
                pool_v=pool_v, pool_dtype=kvdt, req_to_token=r2t, req_pool_idx=rows, seq_lens=lens,
                full_to_swa=mapping if use_map else None, window=window, sinks=s)
    return args, codecs.decode_store(q, qdt), codecs.decode_store(kd, kvdt), codecs.decode_store(vd, kvdt)


def textbook_causal(q, k, v, scale):
    """Full causal attention as matrices: softmax(QK^T * scale + triangular mask) V."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    out = np.empty_like(q)
    mask = np.triu(np.ones((T, T), dtype=bool), 1)
    for h in range(Hq):
        s = scale * q[:, h, :] @ k[:, h // G, :].T
        s[mask] = -np.inf
        out[:, h, :] = scipy.special.softmax(s, axis=1) @ v[:, h // G, :]
    return out


@pytest.mark.parametrize("window", [-1, 40, 41, 1000])
def test_window_at_least_T_is_full_causal(window):
    rng = np.random.default_rng(7)
    T, Hq, Hkv, D = 40, 4, 2, 16
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, window, P=4, sinks=False)
    got = O.extend(**args)
    want = textbook_causal(q, k, v, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-13)


def test_sink_minus_inf_is_plain_softmax():
    rng = np.random.default_rng(8)
    T, Hq, Hkv, D, W = 30, 4, 4, 8, 5
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, W, P=2, margin=3, sinks=False)
    no_sink = O.extend(**args)
    args["sinks"] = np.full(Hq, -np.inf)
    with_inf = O.extend(**args)
    assert np.array_equal(no_sink, with_inf)
    scale = 1 / math.sqrt(D)
    for i in range(T):
        lo = max(0, i - W)
        for h in range(Hq):
            p = scipy.special.softmax(scale * k[lo:i + 1, h, :] @ q[i, h, :])
            np.testing.assert_allclose(no_sink[i, h], p @ v[lo:i + 1, h, :], rtol=1e-12, atol=1e-14)


def brute_force(q, k, v, sinks, window, scale):
    """Pure-Python loops with math.exp, one (query, head) at a time."""
    T, Hq, D = len(q), len(q[0]), len(q[0][0])
    G = Hq // len(k[0])
    out = [[[0.0] * D for _ in range(Hq)] for _ in range(T)]
    for i in range(T):
        lo = 0 if window < 0 else max(0, i - window)
        for h in range(Hq):
            g = h // G
            scores = []
            for j in range(lo, i + 1):
                scores.append(scale * sum(q[i][h][d] * k[j][g][d] for d in range(D)))
            sig = -math.inf if sinks is None else sinks[h]
            m = max(max(scores), sig)
            ws = [math.exp(s - m) for s in scores]
            den = sum(ws) + (0.0 if sinks is None else math.exp(sig - m))
            for d in range(D):
                out[i][h][d] = sum(w * v[lo + n][g][d] for n, w in enumerate(ws)) / den
    return np.array(out)


@pytest.mark.parametrize("T", [1, 2, 5, 8])
@pytest.mark.parametrize("window", [0, 1, 2, 8])
@pytest.mark.parametrize("sinks", [True, False])
def test_brute_force_tiny(T, window, sinks):
    rng = np.random.default_rng(100 * T + 10 * window + sinks)
    Hq, Hkv, D = 4, 2, 4
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, window, P=1, sinks=sinks)
    got = O.extend(**args)
    want = brute_force(q.tolist(), k.tolist(), v.tolist(), None if args["sinks"] is None else list(args["sinks"]),
                       window, 1 / math.sqrt(D))
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_window_zero_closed_form():
    rng = np.random.default_rng(9)
    T, Hq, Hkv, D = 12, 2, 2, 8
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, 0, P=2)
    got = O.extend(**args)
    s = np.einsum("thd,thd->th", q, k) / math.sqrt(D)
    sig = 1 / (1 + np.exp(-(s - args["sinks"][None, :])))
    np.testing.assert_allclose(got, v * sig[:, :, None], rtol=1e-12, atol=1e-15)
    args["sinks"] = None
    got = O.extend(**args)
    assert np.array_equal(got, v)  # exactly v_i: a single key with weight 1


def test_identical_keys_closed_form():
    rng = np.random.default_rng(10)
    T, Hq, Hkv, D, W = 20, 2, 1, 8, 6
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, W, P=4, margin=2)
    krow = rng.standard_normal(D).astype(np.float32).astype(np.float64)
    pool_k = args["pool_k"].copy()
    used = np.isfinite(pool_k[:, 0, 0])
    pool_k[used] = krow.astype(np.float32)
    args["pool_k"] = pool_k
    got = O.extend(**args)
    for i in range(T):
        lo = max(0, i - W)
        n = i - lo + 1
        for h in range(Hq):
            s = float(q[i, h] @ krow) / math.sqrt(D)
            want = v[lo:i + 1, 0].mean(axis=0) * n / (n + math.exp(args["sinks"][h] - s))
            np.testing.assert_allclose(got[i, h], want, rtol=1e-12, atol=1e-14)


def test_gqa_equals_expanded_heads():
    """G q heads sharing one kv head equal G copies of that kv head with G = 1."""
    rng = np.random.default_rng(11)
    T, Hq, Hkv, D, W = 16, 8, 2, 8, 5
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, W, P=2, margin=1)
    got = O.extend(**args)
    G = Hq // Hkv
    args["pool_k"] = np.repeat(args["pool_k"], G, axis=1)
    args["pool_v"] = np.repeat(args["pool_v"], G, axis=1)
    assert np.array_equal(O.extend(**args), got)


def test_decode_matches_last_extend_row_and_dequant_scale():
    rng = np.random.default_rng(12)
    T, Hq, Hkv, D, W = 25, 4, 2, 8, 7
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, W, P=4, margin=4, kvdt="e4m3", qdt="bf16")
    full = O.extend(**args)
    dec = O.decode(args["q"][T - 1:T], "bf16", args["pool_k"], args["pool_v"], "e4m3", args["req_to_token"],
                   args["req_pool_idx"], args["seq_lens"], args["full_to_swa"], W, args["sinks"])
    assert np.array_equal(dec[0], full[T - 1])
    # k_scale multiplies every logit; v_scale multiplies the output linearly
    d2 = O.decode(args["q"][T - 1:T], "bf16", args["pool_k"], args["pool_v"], "e4m3", args["req_to_token"],
                  args["req_pool_idx"], args["seq_lens"], args["full_to_swa"], W, args["sinks"], v_scale=2.0)
    np.testing.assert_allclose(d2, 2 * dec, rtol=1e-14)
    d3 = O.decode(args["q"][T - 1:T], "bf16", args["pool_k"], args["pool_v"], "e4m3", args["req_to_token"],
                  args["req_pool_idx"], args["seq_lens"], args["full_to_swa"], W, args["sinks"],
                  scale=2 / math.sqrt(D))
    d4 = O.decode(args["q"][T - 1:T], "bf16", args["pool_k"], args["pool_v"], "e4m3", args["req_to_token"],
                  args["req_pool_idx"], args["seq_lens"], args["full_to_swa"], W, args["sinks"], k_scale=2.0)
    np.testing.assert_allclose(d3, d4, rtol=1e-13)


def test_in_window_tombstone_raises():
    rng = np.random.default_rng(13)
    args, *_ = dense_case(rng, 20, 2, 2, 4, 4, P=2, margin=0, evict=True)
    dec = [args[k] for k in ("pool_k", "pool_v", "pool_dtype", "req_to_token", "req_pool_idx", "seq_lens",
                             "full_to_swa")]
    q_last = args["q"][19:20]
    out = O.decode(q_last, "f32", *dec, 4, args["sinks"])
    assert np.isfinite(out).all()
    with pytest.raises(O.OracleError):
        O.decode(q_last, "f32", *dec, 12, args["sinks"])  # reaches into evicted pages
    with pytest.raises(O.OracleError):
        O.extend(**args)  # early queries of a prefill see evicted pages


def test_pair_count_ratio_matches_page_claim():
    g = golden()["swa_cost_ratio"]
    T, W = g["T"], g["W"]
    swa = O.scored_pairs(T, W)
    full = O.scored_pairs(T, -1)
    assert full == T * (T + 1) // 2
    assert swa == T * (W + 1) - W * (W + 1) // 2
    ratio = swa / full
    assert ratio < g["fraction_below"]
    assert abs(ratio / (2 * W / T) - 1) < 0.01  # about 2W/T
    assert O.scored_pairs(10, 20) == O.scored_pairs(10, -1)


def test_layout_invariance_of_oracle():
    """The same logical K/V stored under another slot permutation gives the same output."""
    rng = np.random.default_rng(14)
    args1, q, k, v = dense_case(np.random.default_rng(15), 30, 4, 2, 8, 6, P=2, margin=2)
    args2, *_ = dense_case(np.random.default_rng(16), 30, 4, 2, 8, 6, P=2, margin=2)
    args2["q"], args2["sinks"] = args1["q"], args1["sinks"]
    # rebuild pool 2 from the logical values of case 1
    for name, arr in (("pool_k", k), ("pool_v", v)):
        pool = np.full_like(args2[name], np.nan)
        for j in range(30):
            slot = args2["full_to_swa"][args2["req_to_token"][1, j]]
            if slot > 0:
                pool[slot] = arr[j].astype(np.float32)
        args2[name] = pool
    assert np.array_equal(O.extend(**args1), O.extend(**args2))
    del rng


# ---------------------------------------------------------------------------
# planted mistakes: each plausible error in the attention oracle trips a pin
# ---------------------------------------------------------------------------


@pytest.mark.parametrize("mutation", ["drop_sink", "no_scale", "scaled_output"])
def test_pins_catch_planted_mistakes(monkeypatch, mutation):
    original = O.attend

    def mutant(q, keys, values, sink, scale):
        if mutation == "drop_sink":
            return original(q, keys, values, None, scale)
        if mutation == "no_scale":
            return original(q, keys, values, sink, 1.0)
        return original(q, keys, values, sink, scale) * 1.01

    monkeypatch.setattr(O, "attend", mutant)
    rng = np.random.default_rng(17)
    args, q, k, v = dense_case(rng, 5, 4, 2, 4, 2, P=1, sinks=True)
    got = O.extend(**args)
    want = brute_force(q.tolist(), k.tolist(), v.tolist(), list(args["sinks"]), 2, 1 / math.sqrt(4))
    assert not np.allclose(got, want, rtol=1e-9, atol=1e-12)


def test_pins_catch_off_by_one_window(monkeypatch):
    real_attention = O.attention

    def shifted(*a, **kw):
        kw = dict(kw)
        if "window" in kw:
            kw["window"] = kw["window"] - 1
        return real_attention(*a, **kw)

    rng = np.random.default_rng(18)
    args, q, k, v = dense_case(rng, 8, 2, 2, 4, 2, P=1, sinks=True)
    want = brute_force(q.tolist(), k.tolist(), v.tolist(), list(args["sinks"]), 2, 0.5)
    a = dict(args)
    args_pos = (a.pop("q"), a.pop("q_dtype"), a.pop("pool_k"), a.pop("pool_v"), a.pop("pool_dtype"),
                a.pop("req_to_token"), a.pop("req_pool_idx"), a.pop("seq_lens"), a.pop("full_to_swa"))
    got = shifted(*args_pos, window=a["window"], sinks=a["sinks"], prefix_lens=a["prefix_lens"],
                  qo_indptr=a["qo_indptr"])
    assert not np.allclose(got, want, rtol=1e-9, atol=1e-12)
    good = real_attention(*args_pos, window=a["window"], sinks=a["sinks"], prefix_lens=a["prefix_lens"],
                          qo_indptr=a["qo_indptr"])
    np.testing.assert_allclose(good, want, rtol=1e-12, atol=1e-14)


# ---------------------------------------------------------------------------
# validate: a hand-built batch whose violations are counted by hand
# (page 2; full pool 8 rows + page 0 -> mapping of 11 entries ending in -1;
# SWA pool 6 rows).
# ---------------------------------------------------------------------------

def hand_built_batch():
    mapping = np.zeros(11, dtype=np.int64)
    mapping[-1] = -1
    mapping[[2, 3, 4, 5, 6, 7, 8]] = [2, 3, 4, 0, -1, 9, 5]  # 5: tombstone, 6: planted -1, 7: slot past the pool
    r2t = np.zeros((4, 6), dtype=np.int32)
    r2t[1] = [2, 3, 4, 5, 6, 7]
    r2t[2] = [2, 3, 99, 8, -1, 4]  # 99: past the mapping; -1 reads the sentinel
    r2t[3] = 8
    rows = np.array([1, 2, 7, 3, 0, 1], dtype=np.int32)  # 7: no such row
    lens = np.array([6, 5, 3, 7, 3, 2], dtype=np.int32)  # 7: longer than a row
    store = np.array([2, 3, 3, 0, 0, 1, 7, -1, 5, 5, 5], dtype=np.int64)
    return mapping, r2t, rows, lens, store


HAND_COUNTS = {
    # decode, W = 2, with the mapping (SWA pool of 6 rows)
    "decode": dict(bad_requests=2, positions=11, full_out_of_range=1, tombstones=4, sentinels=2,
                   slot_out_of_range=1, store_locs=11, store_out_of_range=2, store_duplicates=3, qo_bad=0),
    # extend, W = 2, prefixes [4, 5, 0, 0, 1, 3] (the last one exceeds its length)
    "extend": dict(bad_requests=3, positions=9, full_out_of_range=0, tombstones=4, sentinels=2,
                   slot_out_of_range=1, store_locs=0, store_out_of_range=0, store_duplicates=0, qo_bad=0),
    # full layer (no mapping), W = -1, full pool of 10 rows
    "full": dict(bad_requests=2, positions=16, full_out_of_range=0, tombstones=3, sentinels=0,
                 slot_out_of_range=2, store_locs=0, store_out_of_range=0, store_duplicates=0, qo_bad=0),
}
EXTEND_PREFIX = np.array([4, 5, 0, 0, 1, 3], dtype=np.int32)
# Query rows of the extend batch above, 9 rows in all.  New positions per request
# (seq - prefix): 2, 0, bad, 7 (bad), 2, bad.  Rows given: [0, 2) right; [2, 1)
# decreasing (1); [1, 4) a bad request, its count not checked, rows in order;
# [4, 4) for a bad request; [4, 5) one row for two positions (2); [5, 10) past
# total_q = 9 (3).
EXTEND_QO = np.array([0, 2, 1, 4, 4, 5, 10], dtype=np.int32)
EXTEND_QO_BAD = 3


def test_validate_hand_counted():
    mapping, r2t, rows, lens, store = hand_built_batch()
    assert O.validate(r2t, rows, lens, mapping, 2, 6, 2, store_loc=store) == HAND_COUNTS["decode"]
    assert O.validate(r2t, rows, lens, mapping, 2, 6, 2, prefix_lens=EXTEND_PREFIX) == HAND_COUNTS["extend"]
    assert O.validate(r2t, rows, lens, None, -1, 10, 2) == HAND_COUNTS["full"]
    got = O.validate(r2t, rows, lens, mapping, 2, 6, 2, prefix_lens=EXTEND_PREFIX, qo_indptr=EXTEND_QO, total_q=9)
    assert got == dict(HAND_COUNTS["extend"], qo_bad=EXTEND_QO_BAD)


def test_validate_clean_workload_counts_nothing():
    """A generated batch keeps every contract: only positions and locs count."""
    wl = WL.decode_workload("clean", 5, [1, 40, 300], 8, 2, 16, 4, "bf16", "bf16", with_store=True, live_margin=3)
    loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
    c = O.validate(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window, wl.pool_k.shape[0],
                   wl.page_size, store_loc=loc)
    assert c["positions"] == sum(min(n, wl.window + 1) for n in wl.seq_lens)
    assert c["store_locs"] == loc.size
    assert sum(v for k, v in c.items() if k not in ("positions", "store_locs")) == 0


# ---------------------------------------------------------------------------
# evict: hand-worked ranges and a hand-built release, then properties that
# tie it to the attention path ([SWA] 运行时, 双池与映射表)
# ---------------------------------------------------------------------------

def test_evict_range_hand_worked():
    # chunk cache: pre_len - W, aligned down to the page
    assert O.evict_range(1000, 0, 0, 128, 16, 0, 0) == (0, 864)
    # radix cache: pre_len - max(W, P)
    assert O.evict_range(1000, 0, 0, 128, 64, O.RADIX, 0) == (0, 832)
    assert O.evict_range(1000, 0, 0, 16, 64, O.RADIX, 0) == (0, 896)     # max(16, 64) = 64
    # protected prefix raises the lower bound; evicted length too
    assert O.evict_range(1000, 100, 300, 128, 16, 0, 0) == (300, 864)
    # nothing left of the window yet
    assert O.evict_range(100, 0, 0, 128, 16, 0, 0)[1] == 0
    # decode interval: wait until 128 tokens have left the window
    assert O.evict_range(1000, 800, 0, 128, 16, 0, 128) == (800, 800)     # 864 - 800 = 64 < 128
    assert O.evict_range(1056, 800, 0, 128, 16, 0, 128) == (800, 928)    # 928 - 800 = 128


def test_evict_hand_built():
    # page 4, window 4; one request (row 1) of 20 positions on full pages 3,1,4,2,5
    # mapped to SWA pages 7,2,9,4,6 (in-page offsets kept); pre_len 19 -> bound 15 -> 12
    P = 4
    full_pages, swa_pages = [3, 1, 4, 2, 5], [7, 2, 9, 4, 6]
    r2t = np.zeros((2, 20), dtype=np.int32)
    mapping = np.zeros(6 * P + P + 1, dtype=np.int64)
    mapping[-1] = -1
    for j in range(20):
        f = full_pages[j // P] * P + j % P
        r2t[1, j] = f
        mapping[f] = swa_pages[j // P] * P + j % P
    m, ev, pages = O.evict(r2t, [1], mapping, [19], [0], 4, P)
    assert pages.tolist() == [7, 2, 9]
    assert ev.tolist() == [12]
    released = set(r2t[1, :12].tolist())
    for f in range(mapping.size):
        assert m[f] == (0 if f in released else mapping[f])
    # a second release frees nothing and changes nothing
    m2, ev2, pages2 = O.evict(r2t, [1], m, [19], ev, 4, P)
    assert pages2.size == 0 and np.array_equal(m2, m) and ev2.tolist() == [12]


def test_evict_keeps_the_next_window_and_its_attention():
    """After releasing everything left of the current token's window, that
    window has no tombstone and decode gives the very same output."""
    wl = WL.decode_workload("evict", 9, [1, 40, 300, 1000, 129], 8, 2, 128, 16, "bf16", "bf16", sinks=True,
                            live_margin=200)
    before = O.decode(wl.q, "bf16", wl.pool_k, wl.pool_v, "bf16", wl.req_to_token, wl.req_pool_idx, wl.seq_lens,
                      wl.full_to_swa, wl.window, wl.sinks)
    pre = wl.seq_lens.astype(np.int64) - 1
    m, ev, pages = O.evict(wl.req_to_token, wl.req_pool_idx, wl.full_to_swa, pre, np.zeros(5, np.int64), 128, 16)
    assert pages.size > 0 and np.all(pages > 0)
    assert np.unique(pages).size == pages.size                     # each page released once
    after = O.decode(wl.q, "bf16", wl.pool_k, wl.pool_v, "bf16", wl.req_to_token, wl.req_pool_idx, wl.seq_lens,
                     m, wl.window, wl.sinks)                      # raises on an in-window tombstone
    assert np.array_equal(before, after)
    # every released page was mapped before and is mapped nowhere now
    swa_pages_before = set((wl.full_to_swa[wl.full_to_swa > 0] // 16).tolist())
    swa_pages_after = set((m[m > 0] // 16).tolist())
    assert set(pages.tolist()) <= swa_pages_before
    assert not set(pages.tolist()) & swa_pages_after


# ---------------------------------------------------------------------------
# paired allocation ([POOLS] 三重映射, alloc_extend, alloc_decode, 扩容与不足,
# 双池 + 映射表): slot = page * P + offset
# ---------------------------------------------------------------------------

# A batch worked by hand with P = 4 and free list [5, 3, 8, 1, 6, 2, 7]:
#   req 0: prefix 6, seq 15, last_loc 29 (page 7, offset 1 = (6-1) % 4).
#          part 1 fills positions 6, 7 -> 30, 31; it needs ceil(15/4) - ceil(6/4) = 2
#          new pages (5 and 3): positions 8..11 -> 20..23 (page 5), then the tail
#          12..14 -> 12, 13, 14 at the start of its last new page (3).
#   req 1: no prefix (last_loc -1), seq 5: pages 8 and 1 -> 32..35 and 4.
#   req 2: prefix 8 (page aligned, no part 1), seq 9: one page (6) -> 24.
#   req 3: prefix 3, seq 4: the token stays in the half-full page: 38 + 1 = 39.
HAND_ALLOC = dict(pre=[6, 0, 8, 3], seq=[15, 5, 9, 4], last=[29, -1, 11, 38], free=[5, 3, 8, 1, 6, 2, 7], P=4,
                  out=[30, 31, 20, 21, 22, 23, 12, 13, 14, 32, 33, 34, 35, 4, 24, 39], pages=5)


def test_alloc_extend_hand_worked():
    h = HAND_ALLOC
    out, taken = O.alloc_extend(h["pre"], h["seq"], h["last"], h["free"], h["P"])
    assert out.tolist() == h["out"] and taken == h["pages"]
    assert O.pages_needed(h["pre"], h["seq"], h["P"]) == h["pages"]
    # one page fewer on the free list: nothing is allocated
    assert O.alloc_extend(h["pre"], h["seq"], h["last"], h["free"][:4], h["P"]) is None


def _token_by_token(pre_lens, seq_lens, last_loc, free, P):
    """An allocator that walks every new position in order and takes the next
    free page whenever a position starts a page; a position in the page the
    prefix ends in uses that page (the page of last_loc)."""
    out, nxt = [], 0
    for pre, seq, last in zip(pre_lens, seq_lens, last_loc):
        page = last // P if pre % P else None
        for j in range(pre, seq):
            if j % P == 0:
                page = free[nxt]
                nxt += 1
            out.append(page * P + j % P)
    return out, nxt


def _alloc_case(rng, B, P, max_len=300):
    pre = rng.integers(0, max_len, B)
    pre[rng.random(B) < 0.3] = 0
    seq = pre + rng.integers(0, max_len, B)
    # last_loc: a slot of some used page, at the in-page offset of position pre - 1
    last = np.where(pre > 0, (rng.integers(1000, 2000, B)) * P + (pre - 1) % P, -1)
    free = rng.permutation(np.arange(1, 1000))
    return pre, seq, last, free


@pytest.mark.parametrize("P", [1, 2, 4, 16, 64])
def test_alloc_extend_equals_token_by_token(P):
    rng = np.random.default_rng(300 + P)
    for _ in range(20):
        pre, seq, last, free = _alloc_case(rng, int(rng.integers(1, 9)), P)
        if O.pages_needed(pre, seq, P) > free.size:
            continue
        want, taken = _token_by_token(pre.tolist(), seq.tolist(), last.tolist(), free.tolist(), P)
        out, n = O.alloc_extend(pre, seq, last, free, P)
        assert out.tolist() == want and n == taken
        assert np.unique(out).size == out.size and not np.any((out >= 0) & (out < P))   # distinct, never page 0
        pos = np.concatenate([np.arange(p, s) for p, s in zip(pre, seq)])
        assert np.array_equal(out % P, pos % P)                                         # in-page offsets
        assert O.pages_bound(int((seq - pre).sum()), len(pre), P) >= n


def test_pages_bound_hand_worked():
    """The optimistic page bound printed in the Pools article (扩容与不足):
    extend_num_tokens // page_size + batch + 1, worked by hand.  A dropped "+ 1"
    or a ceiling in place of the floor changes every value below."""
    assert O.pages_bound(230, 3, 16) == 18        # 230 // 16 = 14; 14 + 3 + 1
    assert O.pages_bound(2048, 1, 64) == 34       # 32 + 1 + 1
    assert O.pages_bound(524288, 256, 64) == 8449  # 8192 + 256 + 1 (one 2048-token chunk each)
    assert O.pages_bound(15, 1, 16) == 2          # 0 + 1 + 1: the floor, not the ceiling
    assert O.pages_bound(0, 0, 16) == 1


def test_alloc_page_size_one_slices_the_free_list():
    rng = np.random.default_rng(311)
    pre, seq, last, free = _alloc_case(rng, 6, 1)
    n = int((seq - pre).sum())
    out, taken = O.alloc_extend(pre, seq, last, free, 1)
    assert out.tolist() == free[:n].tolist() and taken == n


@pytest.mark.parametrize("P", [1, 4, 64])
def test_alloc_decode_is_extend_of_one_token(P):
    rng = np.random.default_rng(320 + P)
    seq = rng.integers(1, 500, 40)
    seq[:4] = [1, P, P + 1, 2 * P]
    last = np.where(seq > 1, rng.integers(1000, 2000, 40) * P + (seq - 2) % P, -1)
    free = rng.permutation(np.arange(1, 500))
    dec, n_dec = O.alloc_decode(seq, last, free, P)
    ext, n_ext = O.alloc_extend(seq - 1, seq, last, free, P)
    assert dec.tolist() == ext.tolist() and n_dec == n_ext == int(np.sum((seq - 1) % P == 0))


def test_alloc_paired_offsets_mapping_and_sentinel():
    P = 16
    rng = np.random.default_rng(330)
    B = 6
    pre = np.array([0, 5, 16, 31, 100, 0])
    seq = pre + np.array([40, 11, 1, 33, 0, 16])
    n_full = 64 * P
    mapping = np.zeros(n_full + P + 1, np.int64)
    mapping[-1] = -1
    # existing prefixes: full page fp <-> SWA page sp, same offsets
    last = np.full(B, -1)
    for b in range(B):
        if pre[b]:
            fp, sp = 40 + b, 20 + b
            last[b] = fp * P + (pre[b] - 1) % P
            mapping[fp * P:(fp + 1) * P] = sp * P + np.arange(P)
    full_free = rng.permutation(np.arange(1, 40))
    swa_free = rng.permutation(np.arange(1, 20))
    full, swa, m, taken = O.alloc_paired(pre, seq, last, full_free, swa_free, mapping, P)
    assert full.size == swa.size == int((seq - pre).sum())
    assert np.array_equal(full % P, swa % P)
    assert np.array_equal(m[full], swa)
    untouched = np.ones(m.size, bool)
    untouched[full] = False
    assert np.array_equal(m[untouched], mapping[untouched]) and m[-1] == -1
    # the SWA side continued from the mapped last_loc, e.g. request 1's first token
    assert swa[40] == mapping[last[1]] + 1
    # either free list too short: nothing
    need = O.pages_needed(pre, seq, P)
    assert O.alloc_paired(pre, seq, last, full_free, swa_free[:need - 1], mapping, P) is None


def test_alloc_pins_catch_floor_for_ceil(monkeypatch):
    monkeypatch.setattr(O, "_ceil_div", lambda a, b: a // b)
    h = HAND_ALLOC
    got = O.alloc_extend(h["pre"], h["seq"], h["last"], h["free"], h["P"])
    assert got is None or got[0].tolist() != h["out"]


# ---------------------------------------------------------------------------
# unified pool ([PR] 实现拆解: page-major envelope, dense per-layer views,
# kernel-facing ids)
# ---------------------------------------------------------------------------

def _envelope_raw(rng, layer_num, H, D, P, num_pages, anchor=0, pad=True):
    """A raw byte buffer whose every envelope row holds its own random bytes,
    placed row by row with the envelope formula; returns (raw, rows) with
    rows[(page, layer, kv, off)] the bytes placed there."""
    g = O.unified_geometry(layer_num, H, D, 2, P, num_pages)
    raw = np.zeros(anchor + g["total_bytes"] + (g["tail_pad"] if pad else 0), dtype=np.uint8)
    rows = {}
    for page in range(num_pages):
        for layer in range(layer_num):
            for kv in (0, 1):
                for off in range(P):
                    at = O.envelope_offset(anchor, page, layer, kv, off, layer_num, g["row_bytes"], P)
                    row = rng.integers(0, 256, g["row_bytes"], dtype=np.uint8)
                    raw[at:at + g["row_bytes"]] = row
                    rows[(page, layer, kv, off)] = row
    return raw, rows, g


def test_unified_view_addressing_equals_envelope():
    L, H, D, P, pages, anchor = 3, 2, 8, 4, 5, 96
    row_bytes = H * D * 2
    v2p = np.array([0, 3, 1, 4, 2])            # virtual page -> physical page
    for t in range(len(v2p) * P):
        kid = int(O.unified_kernel_ids([t], v2p, P, 2 * L)[0])
        for layer in range(L):
            for kv in (0, 1):
                via_view = O.unified_view_base(anchor, layer, kv, row_bytes, P) + kid * row_bytes
                assert via_view == O.envelope_offset(anchor, v2p[t // P], layer, kv, t % P, L, row_bytes, P)


def test_unified_strided_views_match_placed_rows_byte_for_byte():
    rng = np.random.default_rng(400)
    L, H, D, P, pages, anchor = 3, 2, 8, 4, 6, 64
    raw, rows, g = _envelope_raw(rng, L, H, D, P, pages, anchor)
    ks, vs = O.unified_views(raw, anchor, L, H, D, np.uint16, P, pages)
    v2p = rng.permutation(pages)
    for t in range(pages * P):
        kid = int(O.unified_kernel_ids([t], v2p, P, 2 * L)[0])
        for layer in range(L):
            for kv, views in ((0, ks), (1, vs)):
                got = np.ascontiguousarray(views[layer][kid]).view(np.uint8).ravel()
                assert np.array_equal(got, rows[(int(v2p[t // P]), layer, kv, t % P)])


def test_unified_tail_pad_is_one_envelope_and_needed():
    rng = np.random.default_rng(401)
    L, H, D, P, pages = 2, 1, 4, 4, 3
    raw, _, g = _envelope_raw(rng, L, H, D, P, pages, pad=False)
    with pytest.raises(O.OracleError):
        O.unified_views(raw, 0, L, H, D, np.uint16, P, pages)     # the last views run past the envelopes
    last_end = O.unified_view_base(0, L - 1, 1, g["row_bytes"], P) + g["n_rows"] * g["row_bytes"]
    assert last_end == g["total_bytes"] + (2 * L - 1) * P * g["row_bytes"] <= g["total_bytes"] + g["tail_pad"]
    raw2, _, _ = _envelope_raw(rng, L, H, D, P, pages, pad=True)
    O.unified_views(raw2, 0, L, H, D, np.uint16, P, pages)


def test_unified_tombstone_clamps_to_the_sink():
    v2p = np.array([2, -1, 0, 1])
    ids = O.unified_kernel_ids(np.arange(16), v2p, 4, 6)
    assert ids[4:8].tolist() == [0, 0, 0, 0]                    # page 1 tombstoned
    assert ids[:4].tolist() == [48, 49, 50, 51]                   # 2 * (4 * 6) + offset
    m = O.unified_mapping(v2p, 4, 6)
    assert m.size == 17 and m[-1] == -1 and np.array_equal(m[:-1], ids)


def test_unified_pins_catch_multiplier_one():
    rng = np.random.default_rng(402)
    L, H, D, P, pages = 2, 1, 4, 4, 4
    raw, rows, _ = _envelope_raw(rng, L, H, D, P, pages)
    ks, _ = O.unified_views(raw, 0, L, H, D, np.uint16, P, pages)
    v2p = np.arange(pages)
    wrong = 0
    for t in range(pages * P):
        kid = int(O.unified_kernel_ids([t], v2p, P, 1)[0])     # physical ids written into dense rows
        got = np.ascontiguousarray(ks[1][kid]).view(np.uint8).ravel()
        wrong += not np.array_equal(got, rows[(t // P, 1, 0, t % P)])
    assert wrong > 0


def test_unified_attention_equals_two_pool_attention():
    """The same logical K/V laid out in a two-pool SWA layer and in a unified
    envelope give exactly the same window attention."""
    rng = np.random.default_rng(403)
    L, H, D, P, W = 2, 2, 8, 4, 5
    lens = np.array([9, 14, 3])
    n_vpages = 1 + sum(-(-int(t) // P) for t in lens)
    vpages = 1 + rng.permutation(n_vpages - 1)               # virtual pages of the requests, page 0 padding
    r2t = np.zeros((4, 16), np.int32)
    at = 0
    for b, t in enumerate(lens):
        npg = -(-int(t) // P)
        for j in range(int(t)):
            r2t[b + 1, j] = vpages[at + j // P] * P + j % P
        at += npg
    v2p = np.concatenate([[0], 1 + rng.permutation(n_vpages - 1)])   # virtual -> physical page
    raw, _, g = _envelope_raw(rng, L, H, D, P, n_vpages)
    # keep the stored bits finite bf16 values: clear the exponent's top bit of every element
    raw_bits = raw.view(np.uint16)
    raw_bits &= np.uint16(0xBFFF)
    ks, vs = O.unified_views(raw, 0, L, H, D, np.uint16, P, n_vpages)
    m_unified = O.unified_mapping(v2p, P, 2 * L)
    # two-pool form: an SWA pool whose slot s = virtual id holds the same rows
    q = codecs.f64_to_bf16_bits(rng.standard_normal((3, 4, D)))
    sinks = rng.standard_normal(4)
    n_virt = n_vpages * P
    identity = np.concatenate([np.arange(n_virt), [-1]]).astype(np.int64)
    for layer in range(L):
        kid = m_unified[:-1]
        pool_k = np.asarray(ks[layer])[kid]
        pool_v = np.asarray(vs[layer])[kid]
        a = O.decode(q, "bf16", ks[layer], vs[layer], "bf16", r2t, np.arange(1, 4), lens, m_unified, W, sinks)
        b = O.decode(q, "bf16", pool_k, pool_v, "bf16", r2t, np.arange(1, 4), lens, identity, W, sinks)
        assert np.array_equal(a, b)


# ---------------------------------------------------------------------------
# chunked local attention ([SWA] 设计: Llama4's chunked local layers) and the
# per-request SWA ring ([POOLS] SWATokenToKVPoolAllocator)
# ---------------------------------------------------------------------------

def masked_matrix(q, k, v, scale, window=-1, chunk=0, sinks=None):
    """Attention as matrices: query i may see key j iff j <= i, j >= i - W
    (W >= 0) and j lies in i's chunk (j // C == i // C, C > 0); a sink adds a
    logit column with no value."""
    T, Hq, D = q.shape
    G = Hq // k.shape[1]
    i = np.arange(T)[:, None]
    j = np.arange(T)[None, :]
    ok = j <= i
    if window >= 0:
        ok &= j >= i - window
    if chunk > 0:
        ok &= (j // chunk) == (i // chunk)
    out = np.empty_like(q)
    for h in range(Hq):
        s = scale * q[:, h, :] @ k[:, h // G, :].T
        s = np.where(ok, s, -np.inf)
        if sinks is not None:
            s = np.concatenate([s, np.full((T, 1), sinks[h])], axis=1)
        p = scipy.special.softmax(s, axis=1)
        out[:, h, :] = p[:, :T] @ v[:, h // G, :]
    return out


@pytest.mark.parametrize("chunk", [40, 41, 1000])
def test_chunk_at_least_T_is_full_causal(chunk):
    rng = np.random.default_rng(500)
    T, Hq, Hkv, D = 40, 4, 2, 16
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, -1, P=4, sinks=False)
    got = O.extend(**args, chunk=chunk)
    np.testing.assert_allclose(got, textbook_causal(q, k, v, 1 / math.sqrt(D)), rtol=1e-12, atol=1e-13)


def test_chunk_one_is_the_window_zero_closed_form():
    rng = np.random.default_rng(501)
    T, Hq, Hkv, D = 12, 2, 2, 8
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, -1, P=2)
    got = O.extend(**args, chunk=1)
    s = np.einsum("thd,thd->th", q, k) / math.sqrt(D)
    sig = 1 / (1 + np.exp(-(s - args["sinks"][None, :])))
    np.testing.assert_allclose(got, v * sig[:, :, None], rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("chunk", [4, 7, 16])
@pytest.mark.parametrize("window", [-1, 3, 10])
def test_chunked_local_matches_the_block_mask(chunk, window):
    rng = np.random.default_rng(510 + chunk + window)
    T, Hq, Hkv, D = 37, 4, 2, 8
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, window, P=4)
    got = O.extend(**args, chunk=chunk)
    want = masked_matrix(q, k, v, 1 / math.sqrt(D), window, chunk, args["sinks"])
    np.testing.assert_allclose(got, want, rtol=1e-12, atol=1e-14)


def test_chunked_local_pair_count():
    # without a window, a chunk of n positions scores n (n + 1) / 2 pairs
    for T, C in ((100, 8), (64, 64), (1000, 96), (7, 3)):
        pairs = sum(i - O.first_key(i, -1, C) + 1 for i in range(T))
        sizes = [C] * (T // C) + ([T % C] if T % C else [])
        assert pairs == sum(n * (n + 1) // 2 for n in sizes)


def test_ring_rows_and_capacity():
    assert O.ring_rows(129, 16) == 144 and O.ring_rows(128, 16) == 128 and O.ring_rows(5, 1) == 5
    assert O.ring_capacity(8, 129, 16) == 8 * 144


@pytest.mark.parametrize("W,n_new,P", [(128, 1, 16), (20, 9, 4), (0, 1, 1), (7, 33, 8)])
def test_ring_positions_of_one_step_never_share_a_row(W, n_new, P):
    """The positions one step reads or writes (the window of its first new
    query through its last) span W + n_new; a ring of that size rounded to a
    page keeps them on distinct rows, and rows of different requests never
    meet.  One row fewer collides."""
    span = W + n_new
    R = O.ring_rows(span, P)
    for row in (1, 2, 5):
        for start in range(0, 3 * R):
            slots = [O.ring_slot(row, j, R) for j in range(start, start + span)]
            assert len(set(slots)) == span
            assert all(row * R <= s < (row + 1) * R for s in slots)
    if span > 1:
        short = span - 1
        slots = [O.ring_slot(1, j, short) for j in range(span)]
        assert len(set(slots)) < span


def test_ring_attention_equals_two_pool_attention():
    rng = np.random.default_rng(520)
    T, Hq, Hkv, D, W = 30, 4, 2, 8, 6
    args, q, k, v = dense_case(rng, T, Hq, Hkv, D, W, P=2, margin=1)
    R = O.ring_rows(T, 4)          # extend of every position: the ring holds them all
    rows = args["req_pool_idx"]
    ring = O.ring_req_to_token(args["req_to_token"].shape[0], args["req_to_token"].shape[1], R)
    n_rows = ring.max() + 1
    pk = np.full((n_rows, Hkv, D), np.nan, dtype=np.float32)
    pv = np.full((n_rows, Hkv, D), np.nan, dtype=np.float32)
    for j in range(T):
        pk[ring[rows[0], j]] = codecs.encode_store(k[j], "f32")
        pv[ring[rows[0], j]] = codecs.encode_store(v[j], "f32")
    want = O.extend(**args)
    ring_args = dict(args, pool_k=pk, pool_v=pv, req_to_token=ring, full_to_swa=None)
    assert np.array_equal(O.extend(**ring_args), want)
