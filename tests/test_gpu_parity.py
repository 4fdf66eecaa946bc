"""GPU parity: the HIP path (through the C ABI) against the CPU oracle on the
same seeded inputs.  Bit-exact for index translation and stores; attention
within max|err| / RMS(oracle) of 1e-5 (f32), 2e-2 (bf16 K/V), 6e-2 (e4m3 K/V),
checked on the kernel's f32 output; the bf16 output must equal the f32 output
rounded to nearest even, bit for bit."""

import numpy as np
import pytest
import torch

from oracle import codecs
from oracle import swa_oracle as O
from sliding_window_attention_swa_amd import workloads as WL

from gpu_path import (TOL, DeviceWorkload, bits_to_device, check, device_to_bits, oracle_decode, oracle_extend,
                      oracle_pools_after_store, run_decode, run_decode_store, run_extend, run_store, say)

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module", autouse=True)
def _gpu():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    from sliding_window_attention_swa_amd import swa  # noqa: F401  (fails loudly if libswa.so is missing)
    yield
    torch.cuda.synchronize()


def bf16_of(t: torch.Tensor) -> np.ndarray:
    return device_to_bits(t.float().to(torch.bfloat16))


# ---------------------------------------------------------------------------
# index translation and stores: bit-exact
# ---------------------------------------------------------------------------


def test_translate_loc_bit_exact():
    from sliding_window_attention_swa_amd import swa
    wl = WL.decode_workload("tl", 11, [300, 40, 1000], 4, 2, 128, 16, "bf16", "bf16")
    rng = np.random.default_rng(0)
    full = wl.req_to_token[1:, :].ravel()
    full = np.concatenate([full[full > 0], [-1, 0, 0, -1]])
    rng.shuffle(full)
    full = full.astype(np.int64)
    say(f"translate_loc n={full.size}")
    m = torch.from_numpy(wl.full_to_swa).cuda()
    out = torch.empty(full.size, dtype=torch.int64, device="cuda")
    swa.swa_translate_loc(torch.from_numpy(full).cuda(), m, out)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), O.translate_loc(full, wl.full_to_swa))
    # indices outside the table become 0 (the padding row), never an out-of-bounds read
    bad = torch.tensor([-5, wl.full_to_swa.size - 1, wl.full_to_swa.size + 7, 1 << 40], dtype=torch.int64).cuda()
    out = torch.empty_like(bad)
    swa.swa_translate_loc(bad, m, out)
    torch.cuda.synchronize()
    assert out.cpu().tolist() == [0, 0, 0, 0]


@pytest.mark.parametrize("window", [128, 0, 7, -1])
@pytest.mark.parametrize("extend", [False, True])
def test_translate_window_bit_exact(window, extend):
    from sliding_window_attention_swa_amd import swa
    say(f"translate_window window={window} extend={extend}")
    if extend:
        wl = WL.extend_workload("tw", 12, [0, 5, 300, 1000], [20, 1, 70, 300], 4, 2, window, 16)
        pre = wl.prefix_lens
    else:
        wl = WL.decode_workload("tw", 12, [1, 2, 129, 130, 700], 4, 2, max(window, 0) if window >= 0 else 128, 16,
                                "bf16", "bf16")
        pre = None
    dw = DeviceWorkload(wl)
    for use_map in (True, False):
        if window < 0 and use_map and not extend:
            continue
        table_ref, indptr_ref = O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens,
                                               wl.full_to_swa if use_map else None, window, prefix_lens=pre)
        table = torch.full((table_ref.size + 5,), -77, dtype=torch.int32, device="cuda")
        indptr = torch.empty(wl.batch + 1, dtype=torch.int32, device="cuda")
        swa.swa_translate_window(dw.index, window, table, indptr, prefix_lens=dw.prefix, use_map=use_map)
        torch.cuda.synchronize()
        t = table.cpu().numpy()
        assert np.array_equal(indptr.cpu().numpy(), indptr_ref)
        assert np.array_equal(t[:table_ref.size], table_ref)
        assert np.all(t[table_ref.size:] == -77)  # nothing written past the windows


def test_translate_window_capacity_and_empty_batch():
    from sliding_window_attention_swa_amd import swa
    wl = WL.decode_workload("cap", 13, [50, 300], 4, 2, 128, 16, "bf16", "bf16")
    dw = DeviceWorkload(wl)
    table = torch.full((60,), -5, dtype=torch.int32, device="cuda")  # smaller than 50 + 129 entries
    guard = torch.full((64,), -5, dtype=torch.int32, device="cuda")
    indptr = torch.empty(3, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(dw.index, 128, table, indptr)
    torch.cuda.synchronize()
    ref, ref_ptr = O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, 128)
    assert np.array_equal(indptr.cpu().numpy(), ref_ptr)
    assert np.array_equal(table.cpu().numpy(), ref[:60])
    assert np.all(guard.cpu().numpy() == -5)
    # empty batch: indptr = [0]
    empty = swa.IndexTables(dw.r2t, dw.rows[:0], dw.lens[:0], None, 16)  # no window table: no mapping either
    ip = torch.full((1,), 9, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(empty, 128, table, ip)
    torch.cuda.synchronize()
    assert ip.item() == 0


STORE_PAIRS = [("bf16", "bf16"), ("f32", "f32"), ("f32", "bf16"), ("bf16", "e4m3"), ("f32", "e4m3")]


@pytest.mark.parametrize("in_dtype,pool_dtype", STORE_PAIRS)
def test_kv_store_bit_exact(in_dtype, pool_dtype):
    from sliding_window_attention_swa_amd import swa
    say(f"kv_store {in_dtype}->{pool_dtype}")
    rng = np.random.default_rng(14)
    rows, H, D, n = 1000, 8, 128, 300
    base = WL.SparsePool(rows, H, D, pool_dtype, np.arange(0), np.zeros((0, H, D), WL.NP_STORE[pool_dtype]))
    loc = rng.choice(np.arange(1, rows), n, replace=False).astype(np.int64)
    x = rng.standard_normal((n, H, D)).astype(np.float32) * rng.choice([1e-3, 1, 30], (n, 1, 1)).astype(np.float32)
    kn = WL.to_store(x, in_dtype)
    vn = WL.to_store(-2 * x, in_dtype)
    from gpu_path import pool_to_device
    k, v = pool_to_device(base), pool_to_device(base)
    swa.swa_kv_store(swa.KvLayer(k, v), torch.from_numpy(loc).cuda(), bits_to_device(kn, in_dtype),
                     bits_to_device(vn, in_dtype))
    torch.cuda.synchronize()
    ek, ev = O.kv_store(base, base, loc, kn, vn, in_dtype, pool_dtype)
    gk, gv = device_to_bits(k), device_to_bits(v)
    for got, exp in ((gk, ek.dense()), (gv, ev.dense())):
        assert np.array_equal(got.view(np.uint8)[1:], exp.view(np.uint8)[1:])


def test_kv_store_e4m3_every_bf16_pattern():
    """All 65,536 bf16 bit patterns (NaN, inf, subnormals, overflow) through the
    store kernel's e4m3 encoder, against the oracle's table-search encoder."""
    from sliding_window_attention_swa_amd import swa
    H, D = 8, 128
    n = 65536 // (H * D)
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16).reshape(n, H, D)
    rows = n + 8
    loc = np.arange(1, n + 1, dtype=np.int64)
    k = torch.zeros((rows, H, D), dtype=torch.uint8, device="cuda")
    v = torch.zeros((rows, H, D), dtype=torch.uint8, device="cuda")
    kb = bits_to_device(bits, "bf16")
    swa.swa_kv_store(swa.KvLayer(k, v), torch.from_numpy(loc).cuda(), kb, kb)
    torch.cuda.synchronize()
    want = codecs.f64_to_e4m3(codecs.bf16_bits_to_f64(bits))
    got = k.cpu().numpy()[1:n + 1]
    assert np.array_equal(got, want)
    assert np.array_equal(v.cpu().numpy()[1:n + 1], want)


def test_kv_store_skips_out_of_pool_locs():
    from sliding_window_attention_swa_amd import swa
    H, D, rows = 2, 128, 16
    k = torch.zeros((rows, H, D), dtype=torch.bfloat16, device="cuda")
    v = torch.zeros((rows, H, D), dtype=torch.bfloat16, device="cuda")
    loc = torch.tensor([3, -1, rows, 1 << 40], dtype=torch.int64, device="cuda")
    new = torch.ones((4, H, D), dtype=torch.bfloat16, device="cuda")
    swa.swa_kv_store(swa.KvLayer(k, v), loc, new, new)
    torch.cuda.synchronize()
    written = (k.float().abs().sum(dim=(1, 2)) > 0).cpu().numpy()
    assert written.tolist() == [i == 3 for i in range(rows)]


# ---------------------------------------------------------------------------
# decode
# ---------------------------------------------------------------------------

DECODE_CASES = {
    # name: (seq_lens, q_heads, kv_heads, window, page, q_dtype, kv_dtype, sinks)
    "f32_g1": ([1, 100, 700], 4, 4, 128, 1, "f32", "f32", True),
    "f32_g4_w3": ([1, 5, 64, 300], 8, 2, 3, 4, "f32", "f32", True),
    "f32_g8": ([1, 33, 129, 400], 16, 2, 128, 16, "f32", "f32", True),
    "f32_g16_w20": ([2, 19, 250], 32, 2, 20, 4, "f32", "f32", False),
    "bf16_g8": ([1, 2, 129, 130, 1000], 16, 2, 128, 16, "bf16", "bf16", True),
    "bf16_g8_nosink": ([1, 17, 200, 2000], 16, 2, 128, 16, "bf16", "bf16", False),
    "bf16_g1": ([3, 150, 999], 4, 4, 128, 16, "bf16", "bf16", True),
    "bf16_g2": ([3, 150, 999], 8, 4, 128, 16, "bf16", "bf16", True),
    "bf16_g4": ([3, 150, 999], 8, 2, 128, 8, "bf16", "bf16", True),
    "bf16_g16": ([3, 150, 999], 32, 2, 128, 16, "bf16", "bf16", True),
    "bf16_w0": ([1, 9, 500], 16, 2, 0, 16, "bf16", "bf16", True),
    "bf16_w1": ([1, 9, 500], 16, 2, 1, 16, "bf16", "bf16", True),
    "bf16_w300_p64": ([1, 299, 300, 301, 302, 1500], 16, 2, 300, 64, "bf16", "bf16", True),
    # the largest window the one-split window kernel holds (256 keys), and the first past it
    "bf16_w255": ([1, 200, 255, 256, 257, 1200], 16, 2, 255, 16, "bf16", "bf16", True),
    "bf16_w256": ([1, 256, 257, 258, 1200], 16, 2, 256, 16, "bf16", "bf16", True),
    "e4m3_w255_g16": ([256, 2000], 32, 2, 255, 64, "bf16", "e4m3", True),
    "f32_g8_w255": ([1, 256, 300], 16, 2, 255, 16, "f32", "f32", True),
    "e4m3_g8": ([1, 2, 129, 130, 1000], 16, 2, 128, 16, "bf16", "e4m3", True),
    "e4m3_g16_nosink": ([5, 600], 32, 2, 128, 64, "bf16", "e4m3", False),
    # long windows (a per-layer sliding_window_size): split by length as planned by swa_decode_plan
    "bf16_w1023": ([1, 1000, 1023, 1024, 1025, 3000, 5000], 16, 2, 1023, 16, "bf16", "bf16", True),
    "bf16_w4095": ([1, 4000, 4096, 4097, 9000], 16, 2, 4095, 64, "bf16", "bf16", True),
    "e4m3_w4095_g16": ([5, 4097, 7000], 32, 2, 4095, 64, "bf16", "e4m3", True),
    "f32_w1023": ([1, 1024, 2500], 16, 2, 1023, 16, "f32", "f32", True),
    # batches that are a multiple of 8: the window kernel relabels its workgroups across the XCDs
    "bf16_g8_b8": ([1, 130, 2, 129, 900, 17, 128, 3000], 16, 2, 128, 16, "bf16", "bf16", True),
    "e4m3_g8_b16": ([1, 130, 2, 129, 900, 17, 128, 3000, 5, 77, 256, 1000, 129, 130, 131, 64], 16, 2, 128, 64,
                    "bf16", "e4m3", True),
}


@pytest.mark.parametrize("name", list(DECODE_CASES))
def test_decode_small(name):
    lens, hq, hkv, w, P, qd, kvd, sinks = DECODE_CASES[name]
    say(f"decode {name}")
    wl = WL.decode_workload(name, 100 + len(name), lens, hq, hkv, w, P, qd, kvd, sinks=sinks, with_store=True,
                            live_margin=5)
    if kvd == "f32":
        wl.new_k = WL.to_store(codecs.bf16_bits_to_f64(wl.new_k), "f32")
        wl.new_v = WL.to_store(codecs.bf16_bits_to_f64(wl.new_v), "f32")
        wl.new_dtype = "f32"
    dw = DeviceWorkload(wl)
    run_store(dw, wl.new_dtype)
    out = run_decode(dw, "f32")
    ref = oracle_decode(wl)
    check(out, ref, TOL[kvd], name)
    out_bf = run_decode(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


FUSED_CASES = ["bf16_g8", "bf16_g8_nosink", "bf16_g1", "bf16_g2", "bf16_g4", "bf16_g16", "bf16_w0", "bf16_w1",
               "e4m3_g8", "e4m3_g16_nosink", "bf16_w255", "e4m3_w255_g16", "bf16_g8_b8", "e4m3_g8_b16"]


@pytest.mark.parametrize("name", FUSED_CASES)
def test_decode_store_fused(name):
    """swa_decode_store = swa_kv_store + swa_decode: the same pools and the same
    output bits as the two calls, and within tolerance of the oracle."""
    lens, hq, hkv, w, P, qd, kvd, sinks = DECODE_CASES[name]
    say(f"decode+store fused {name}")
    wl = WL.decode_workload(name, 100 + len(name), lens, hq, hkv, w, P, qd, kvd, sinks=sinks, with_store=True,
                            live_margin=5)
    two = DeviceWorkload(wl)
    run_store(two)
    want = run_decode(two, "f32")
    one = DeviceWorkload(wl)
    got = run_decode_store(one, "f32")
    assert np.array_equal(got.cpu().numpy(), want.cpu().numpy())
    for a, b in ((one.layer.k, two.layer.k), (one.layer.v, two.layer.v)):
        assert np.array_equal(device_to_bits(a).view(np.uint8), device_to_bits(b).view(np.uint8))
    check(got, oracle_decode(wl), TOL[kvd], f"fused {name}")
    fused_bf = run_decode_store(DeviceWorkload(wl), "bf16")
    assert np.array_equal(device_to_bits(fused_bf), bf16_of(got))


FULL_CASES = {
    "bf16_full_g16": ([1, 37, 600, 3000], 16, 1, "bf16", "bf16"),
    "bf16_full_g8": ([1, 129, 2500], 16, 2, "bf16", "bf16"),
    "e4m3_full_g8": ([2, 777, 2000], 16, 2, "bf16", "e4m3"),
    "f32_full_g2": ([1, 64, 900], 4, 2, "f32", "f32"),
    "f32_full_g16": ([3, 200, 1100], 32, 2, "f32", "f32"),
}


@pytest.mark.parametrize("name", list(FULL_CASES))
@pytest.mark.parametrize("splits", [None, 1, 3, 8])
def test_decode_full_layer_splits(name, splits):
    """W = -1 (full layer): keys straight from req_to_token, split-K partials
    merged with the sink added once."""
    lens, hq, hkv, qd, kvd = FULL_CASES[name]
    say(f"decode full {name} splits={splits}")
    wl = WL.decode_workload(name, 7 + len(name), lens, hq, hkv, -1, 16, qd, kvd, sinks=True)
    dw = DeviceWorkload(wl)
    out = run_decode(dw, "f32", num_splits=splits)
    ref = oracle_decode(wl)
    check(out, ref, TOL[kvd], f"{name} splits={splits}")
    out_bf = run_decode(dw, "bf16", num_splits=splits)
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


@pytest.mark.parametrize("kvd", ["bf16", "e4m3", "f32"])
def test_decode_full_layer_max_splits(kvd):
    """The largest split count the library accepts (1024): most splits hold no
    key and the merge must ignore them; the workspace is sized by the planner's
    upper bound for this many keys."""
    from sliding_window_attention_swa_amd import swa
    lens = [1, 700, 3000]
    qd = "f32" if kvd == "f32" else "bf16"
    say(f"decode full max splits {kvd}")
    wl = WL.decode_workload("maxsplit", 77, lens, 16, 2, -1, 16, qd, kvd, sinks=True)
    assert swa.lib.swa_decode_workspace_bytes(len(lens), 16, 128, 1 << 20) >= len(lens) * 16 * 1024 * 130 * 4
    out = run_decode(DeviceWorkload(wl), "f32", num_splits=1024)
    check(out, oracle_decode(wl), TOL[kvd], f"max splits {kvd}")


def relabel_swa_pages(wl: WL.Workload, seed: int) -> WL.Workload:
    """Same logical K/V under another SWA page permutation."""
    import copy
    rng = np.random.default_rng(seed)
    P = wl.page_size
    npages = wl.n_swa // P
    perm = np.concatenate([[0], rng.permutation(np.arange(1, npages + 1))])
    w2 = copy.copy(wl)
    m = wl.full_to_swa.copy()
    live = m > 0
    m[live] = perm[m[live] // P] * P + m[live] % P
    w2.full_to_swa = m
    rows = lambda r: perm[r // P] * P + r % P  # noqa: E731
    w2.pool_k = WL.SparsePool(*wl.pool_k.shape, wl.kv_dtype, rows(wl.pool_k.used_rows), wl.pool_k.values)
    w2.pool_v = WL.SparsePool(*wl.pool_v.shape, wl.kv_dtype, rows(wl.pool_v.used_rows), wl.pool_v.values)
    return w2


@pytest.mark.parametrize("kvd", ["bf16", "e4m3"])
def test_decode_layout_invariance(kvd):
    say(f"layout invariance {kvd}")
    wl = WL.decode_workload("inv", 21, [1, 130, 700, 2000], 16, 2, 128, 16, "bf16", kvd)
    a = run_decode(DeviceWorkload(wl), "f32")
    b = run_decode(DeviceWorkload(relabel_swa_pages(wl, 5)), "f32")
    assert torch.equal(a, b)


@pytest.mark.parametrize("window", [1023, 4095])
def test_decode_long_window_planned_splits(window):
    """C2's batch (B = 64, T ~ U[1K, 8K]) with a long window: swa_decode_plan
    splits the window by its length (no hand-passed split count), the split
    partials merge with the sink added once."""
    from sliding_window_attention_swa_amd import swa
    lens = WL.c2_decode_bf16().seq_lens
    wl = WL.decode_workload(f"c2_w{window}", 700 + window, lens, 64, 8, window, 16, "bf16", "bf16", with_store=True)
    splits, ws = swa.swa_decode_plan(wl.batch, 64, 8, 128, window, int(lens.max()))
    say(f"decode c2 lengths, W={window}: {splits} planned splits")
    assert splits > 1 and ws > 0
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_decode(dw, "f32")
    reqs = [0, 1, 17, 40, 63]
    check(out, oracle_decode(wl, only=[(b, h) for b in reqs for h in range(wl.q_heads)]), TOL["bf16"],
          f"W={window} sampled requests")
    out_bf = run_decode(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


@pytest.mark.parametrize("batch,sinks", [(136, True), (160, False)])
def test_decode_e4m3_big_batch_one_wave_per_item(batch, sinks):
    """Batches with more (request, kv head) items than the four-wavefront
    window kernel keeps resident (1024) run e4m3 windows on one wavefront per
    item: ragged lengths (some shorter than the window, one empty), a batch that
    is not a multiple of 8 (plain workgroup order) and one that is (requests
    paired on an XCD), every request against the oracle."""
    rng = np.random.default_rng(batch)
    lens = rng.integers(1, 3000, size=batch)
    lens[:6] = [1, 2, 16, 128, 129, 130]
    wl = WL.decode_workload(f"e4m3_b{batch}", 800 + batch, lens, 64, 8, 128, 64, "bf16", "e4m3", sinks=sinks,
                            with_store=True, live_margin=3)
    say(f"decode e4m3 one wave per item: B={batch}")
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_decode(dw, "f32")
    check(out, oracle_decode(wl), TOL["e4m3"], f"e4m3 B={batch}")
    out_bf = run_decode(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


def test_decode_c1_full_size():
    wl = WL.c1_decode_f32()
    say("decode c1 (1 x 512, f32)")
    out = run_decode(DeviceWorkload(wl), "f32")
    check(out, oracle_decode(wl), TOL["f32"], "c1")


def test_decode_c2_full_size():
    wl = WL.c2_decode_bf16()
    say("decode c2 (64 requests, bf16, with store)")
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_decode(dw, "f32")
    check(out, oracle_decode(wl), TOL["bf16"], "c2")


def test_decode_c5_full_size():
    wl = WL.c5_decode_fp8()
    say("decode c5 (256 requests, e4m3 K/V, with store)")
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_decode(dw, "f32")
    check(out, oracle_decode(wl), TOL["e4m3"], "c5")
    # the stored rows are the oracle's encoding of the new tokens, bit for bit
    loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
    want = codecs.f64_to_e4m3(codecs.bf16_bits_to_f64(wl.new_k))
    assert np.array_equal(dw.k[torch.from_numpy(loc).cuda()].cpu().numpy(), want)


def _pool_rows_equal_oracle_store(wl, dev_pool, oracle_pool):
    """The pool after the store holds the oracle's bytes on every row the
    workload wrote or the store targets, and the NaN fill everywhere else."""
    loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
    rows = np.union1d(oracle_pool.written_rows(), loc[(loc >= 0) & (loc < wl.pool_rows)])
    rows = rows[rows >= wl.page_size]            # page 0 may absorb padded writes
    got = device_to_bits(dev_pool[torch.from_numpy(rows).cuda()])
    assert np.array_equal(got.view(np.uint8), oracle_pool[rows].view(np.uint8))
    nan = WL.NAN_BITS[wl.kv_dtype]
    flat = dev_pool.view(torch.int16) if wl.kv_dtype == "bf16" else dev_pool
    fill = int(np.int16(nan.view(np.int16))) if wl.kv_dtype == "bf16" else int(nan)
    touched = (flat[wl.page_size:] != fill).flatten(1).any(dim=1).sum().item()
    assert touched == rows.size, f"{touched} rows differ from the fill, {rows.size} expected"


def test_decode_store_fused_c2_full_size():
    """The launch the benchmark times, at its timed shape: swa_decode_store on
    C2 (B = 64, a multiple of 8, so the workgroups are relabelled across the
    XCDs and the window table is read speculatively at b * (W + 1)).  f32
    output against the oracle; bf16 output = RNE(f32 output); the pool bytes
    equal the oracle's store."""
    wl = WL.c2_decode_bf16()
    say("decode+store fused c2 (64 requests, bf16)")
    dw = DeviceWorkload(wl)
    out = run_decode_store(dw, "f32")
    check(out, oracle_decode(wl), TOL["bf16"], "c2 fused")
    pk, pv = oracle_pools_after_store(wl)
    _pool_rows_equal_oracle_store(wl, dw.k, pk)
    _pool_rows_equal_oracle_store(wl, dw.v, pv)
    out_bf = run_decode_store(DeviceWorkload(wl), "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


def test_decode_store_fused_c5_full_size():
    """The fused store with e4m3 pools at C5's shape (B = 256): the same pool
    bytes as swa_kv_store + swa_decode and equal to the oracle's encoding; both
    outputs within tolerance of the oracle on sampled requests (every q head).
    (The two calls run this batch on the one-wavefront kernel, whose sums run
    in another order than the fused kernel's, so the bits may differ.)"""
    wl = WL.c5_decode_fp8()
    say("decode+store fused c5 (256 requests, e4m3 K/V)")
    two = DeviceWorkload(wl)
    run_store(two)
    want = run_decode(two, "f32")
    one = DeviceWorkload(wl)
    got = run_decode_store(one, "f32")
    assert torch.equal(one.k, two.k) and torch.equal(one.v, two.v)
    reqs = [0, 7, 8, 100, 201, 255]
    ref = oracle_decode(wl, only=[(b, h) for b in reqs for h in range(wl.q_heads)])
    check(got, ref, TOL["e4m3"], "c5 fused sampled")
    check(want, ref, TOL["e4m3"], "c5 store + decode sampled")
    pk, pv = oracle_pools_after_store(wl)
    _pool_rows_equal_oracle_store(wl, one.k, pk)
    _pool_rows_equal_oracle_store(wl, one.v, pv)


def _c4_oracle_layer(st, ly, q, k, v, reqs):
    """Oracle output of one C4 layer for the requests `reqs` (all q heads),
    from host copies of only the pool rows those requests reference."""
    r2t, rows = st.req_to_token, st.req_pool_idx
    T = int(st.seq_lens[0])
    if ly["kind"] == "full":
        used = np.concatenate([r2t[rows[b], :T] for b in reqs]).astype(np.int64)
        mapping, window = None, -1
    else:
        used = np.concatenate([O.translate_loc(r2t[rows[b], T - 129:T], st.full_to_swa) for b in reqs])
        mapping, window = st.full_to_swa, 128
    used = np.unique(used)
    idx = torch.from_numpy(used).cuda()
    H, D = k.shape[1], k.shape[2]
    pk = WL.SparsePool(k.shape[0], H, D, "bf16", used, device_to_bits(k[idx]))
    pv = WL.SparsePool(v.shape[0], H, D, "bf16", used, device_to_bits(v[idx]))
    only = [(int(b), h) for b in reqs for h in range(st.q_heads)]
    return O.decode(device_to_bits(q), "bf16", pk, pv, "bf16", r2t, rows, st.seq_lens, mapping, window, None,
                    only=only)


def test_mixed_step_c4_full_size_sampled():
    """C4 at full size: the first full layer (W = -1, 4 kv heads, 32K keys,
    split-K as planned for the step) and the first SWA layer (W = 128, 8 kv
    heads, keys through the step's shared window table), against the oracle
    on sampled requests (every q head)."""
    from sliding_window_attention_swa_amd import swa
    st = WL.c4_mixed_step()
    B, Hq, D, T = st.batch, st.q_heads, st.head_dim, int(st.seq_lens[0])
    say("mixed step c4 (B=32, T=32K): one full and one SWA layer — sampled requests")
    index = swa.IndexTables(torch.from_numpy(st.req_to_token).cuda(), torch.from_numpy(st.req_pool_idx).cuda(),
                            torch.from_numpy(st.seq_lens).cuda(), torch.from_numpy(st.full_to_swa).cuda(),
                            st.page_size)
    table = torch.empty(B * 129, dtype=torch.int32, device="cuda")
    indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(index, 128, table, indptr)
    reqs = [0, 13, 31]
    full = next(ly for ly in st.layers if ly["kind"] == "full")
    swl = next(ly for ly in st.layers if ly["kind"] == "swa")
    for ly in (full, swl):
        q, k, v = WL.c4_layer_tensors(st, ly)
        out = torch.empty((B, Hq, D), dtype=torch.float32, device="cuda")
        if ly["kind"] == "full":
            splits, ws_bytes = swa.swa_decode_plan(B, Hq, ly["kv_heads"], D, -1, T)
            assert splits > 1
            ws = torch.empty(ws_bytes // 4, dtype=torch.float32, device="cuda")
            swa.swa_decode(q, swa.KvLayer(k, v), index, -1, out, num_splits=splits, workspace=ws, use_map=False)
        else:
            swa.swa_decode(q, swa.KvLayer(k, v), index, 128, out, slot_table=table, table_indptr=indptr)
        torch.cuda.synchronize()
        ref = _c4_oracle_layer(st, ly, q, k, v, reqs)
        check(out, ref, TOL["bf16"], f"c4 layer {ly['id']} ({ly['kind']})")
        del q, k, v
        torch.cuda.empty_cache()


# ---------------------------------------------------------------------------
# validate (debug report): counts equal the oracle's, exactly
# ---------------------------------------------------------------------------

def _index(r2t, rows, lens, mapping, page):
    from sliding_window_attention_swa_amd import swa
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    return swa.IndexTables(dev(r2t), dev(rows), dev(lens), None if mapping is None else dev(mapping), page)


def test_validate_hand_built_batch():
    from sliding_window_attention_swa_amd import swa
    from test_oracle_pins import EXTEND_PREFIX, HAND_COUNTS, hand_built_batch
    mapping, r2t, rows, lens, store = hand_built_batch()
    say("validate hand-built batch (decode / extend / full layer)")
    ix = _index(r2t, rows, lens, mapping, 2)
    got = swa.swa_validate(ix, 2, 6, store_loc=torch.from_numpy(store).cuda())
    assert got == HAND_COUNTS["decode"]
    got = swa.swa_validate(ix, 2, 6, prefix_lens=torch.from_numpy(EXTEND_PREFIX).cuda())
    assert got == HAND_COUNTS["extend"]
    got = swa.swa_validate(ix, -1, 10, use_map=False)
    assert got == HAND_COUNTS["full"]


def test_validate_planted_violations():
    """A generated decode batch, then tombstones, sentinels, stray indices, a
    bad request and repeated store locations planted into its index data."""
    from sliding_window_attention_swa_amd import swa
    wl = WL.decode_workload("validate", 31, [1, 20, 77, 300, 301, 5], 8, 2, 16, 4, "bf16", "bf16",
                            with_store=True, live_margin=3)
    rng = np.random.default_rng(9)
    r2t, mapping = wl.req_to_token.copy(), wl.full_to_swa.copy()
    rows, lens = wl.req_pool_idx.copy(), wl.seq_lens.astype(np.int32).copy()
    pool_rows, P = wl.pool_k.shape[0], wl.page_size
    loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa)
    say("validate: clean batch, then planted violations")
    clean = swa.swa_validate(_index(r2t, rows, lens, mapping, P), wl.window, pool_rows,
                             store_loc=torch.from_numpy(loc).cuda())
    assert clean == O.validate(r2t, rows, lens, mapping, wl.window, pool_rows, P, store_loc=loc)
    assert clean["tombstones"] == clean["sentinels"] == clean["store_duplicates"] == 0
    # plant: window positions of request 3 (300 tokens) -> tombstone / sentinel / past the pool
    r3 = rows[3]
    fulls = r2t[r3, 300 - 17:300]
    mapping[fulls[0]] = 0
    mapping[fulls[1]] = -1
    mapping[fulls[2]] = pool_rows + 7
    r2t[r3, 300 - 5] = len(mapping) + 100     # past the mapping
    r2t[rows[4], 301 - 2] = -1                  # reads the sentinel
    rows[5] = r2t.shape[0] + 3                  # no such row
    bad_loc = np.concatenate([loc, loc[:3], [pool_rows, -5, 0, 0, 1]]).astype(np.int64)
    rng.shuffle(bad_loc)
    ix = _index(r2t, rows, lens, mapping, P)
    got = swa.swa_validate(ix, wl.window, pool_rows, store_loc=torch.from_numpy(bad_loc).cuda())
    want = O.validate(r2t, rows, lens, mapping, wl.window, pool_rows, P, store_loc=bad_loc)
    assert got == want
    assert want["tombstones"] >= 1 and want["sentinels"] >= 2 and want["slot_out_of_range"] >= 1
    assert want["full_out_of_range"] == 1 and want["bad_requests"] == 1
    # the same data as an extend batch (prefix lengths) and as a full layer
    pre = np.maximum(lens - 40, 0).astype(np.int32)
    got = swa.swa_validate(ix, wl.window, pool_rows, prefix_lens=torch.from_numpy(pre).cuda())
    assert got == O.validate(r2t, rows, lens, mapping, wl.window, pool_rows, P, prefix_lens=pre)
    n_full_rows = len(mapping) - 1
    got = swa.swa_validate(ix, -1, n_full_rows, use_map=False)
    assert got == O.validate(r2t, rows, lens, None, -1, n_full_rows, P)


# ---------------------------------------------------------------------------
# extend
# ---------------------------------------------------------------------------

EXTEND_CASES = {
    # name: (prefix, chunk, q_heads, kv_heads, window, page, sinks)
    "g8_w128": ([0, 5, 300], [33, 100, 70], 16, 2, 128, 16, True),
    "g8_w128_nosink": ([200, 0], [17, 250], 16, 2, 128, 16, False),
    "g8_full": ([0, 40], [50, 17], 16, 2, -1, 8, True),
    "g8_w0": ([10, 0], [20, 5], 16, 2, 0, 4, True),
    "g8_w16": ([100, 3], [64, 33], 16, 2, 16, 16, True),
    "g8_w300": ([50, 700], [400, 31], 16, 2, 300, 64, True),
    "g1": ([20, 300], [40, 90], 2, 2, 128, 16, True),
    "g2": ([20, 300], [40, 90], 4, 2, 128, 16, True),
    "g4": ([20, 300], [40, 90], 8, 2, 128, 16, True),
    "g16": ([20, 300], [40, 90], 32, 2, 128, 16, True),
    "g16_full_one_kv": ([0, 40], [50, 17], 16, 1, -1, 8, True),
    "g16_w300_ragged": ([50, 700, 9], [400, 31, 0], 32, 2, 300, 64, False),
    # ragged batches with requests that add no tokens (one of them with no prefix either)
    "g8_ragged_empty": ([300, 50, 0, 7, 129], [40, 0, 1, 0, 64], 16, 2, 128, 16, True),
    "g4_empty_first": ([64, 0, 500], [0, 0, 200], 8, 2, 128, 16, False),
    "g8_one_token": ([0], [1], 16, 2, 128, 16, True),
    "g8_w255": ([100, 400], [300, 70], 16, 2, 255, 16, True),
    # W = 128 stretches of 1, 2, 3, 4 and 5 steady tiles (whole pairs, an odd last tile)
    "g8_w128_stretches": ([200, 300, 150, 400, 129], [16, 32, 48, 64, 80], 16, 2, 128, 16, True),
    # long bands (W >= 256 and W = -1): the 256-row tiles of the band kernel
    "g8_w256": ([0, 300, 1000], [500, 40, 129], 16, 2, 256, 16, True),
    "g8_w512": ([0, 600, 1500], [700, 300, 64], 16, 2, 512, 16, True),
    "g8_w4095_ragged": ([4100, 10, 0, 5000], [300, 17, 0, 1], 16, 2, 4095, 64, True),
    "g8_full_long": ([3000, 0], [200, 77], 16, 2, -1, 64, False),
    "g1_w1000": ([200, 1500], [300, 40], 2, 2, 1000, 16, True),
    "g2_w600": ([700, 0], [260, 300], 4, 2, 600, 16, True),
    "g4_w2000": ([2500, 100], [150, 400], 8, 2, 2000, 64, False),
    "g16_w1024": ([1200, 33], [100, 260], 32, 2, 1024, 16, True),
}


def test_empty_launches_write_nothing():
    """An extend whose requests add no tokens, and decodes of an empty batch
    (plain and with the fused store): status OK, pools untouched."""
    from sliding_window_attention_swa_amd import swa
    say("empty launches")
    wl = WL.extend_workload("noq", 47, [30, 200], [0, 0], 16, 2, 128, 16)
    dw = DeviceWorkload(wl)
    k0, v0 = dw.k.clone(), dw.v.clone()
    run_store(dw)
    assert run_extend(dw, "f32").shape[0] == 0
    assert run_extend(dw, "bf16", chunk=64).shape[0] == 0
    empty = swa.IndexTables(dw.r2t, dw.rows[:0], dw.lens[:0], None, 16)  # no window table: no mapping either
    out = torch.empty((0, 16, 128), dtype=torch.float32, device="cuda")
    swa.swa_decode(dw.q, dw.layer, empty, 128, out, sinks=dw.sinks)
    swa.swa_decode(dw.q, dw.layer, empty, -1, out, num_splits=4)
    rows = torch.zeros((0, 2, 128), dtype=torch.bfloat16, device="cuda")
    swa.swa_decode_store(dw.q, dw.layer, empty, 128, out, torch.zeros(0, dtype=torch.int64, device="cuda"), rows,
                         rows, sinks=dw.sinks)
    torch.cuda.synchronize()
    assert torch.equal(dw.k.view(torch.int16), k0.view(torch.int16))
    assert torch.equal(dw.v.view(torch.int16), v0.view(torch.int16))


@pytest.mark.parametrize("name", list(EXTEND_CASES))
def test_extend_small(name):
    pre, chunk, hq, hkv, w, P, sinks = EXTEND_CASES[name]
    say(f"extend {name}")
    wl = WL.extend_workload(name, 300 + len(name), pre, chunk, hq, hkv, w, P, sinks=sinks)
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32")
    check(out, oracle_extend(wl), TOL["bf16"], name)
    out_bf = run_extend(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


def test_extend_band_batch_past_request_table():
    """The long-window (band) kernel reads each request's lengths, rows and key
    source into a per-workgroup table for batches of up to 1024 requests; a
    larger batch walks the batch in global memory instead.  1030 requests with
    1-3 new tokens each at W = 300 take that path, checked in full against the
    oracle."""
    say("extend band, 1030 requests (no request table)")
    rng = np.random.default_rng(5)
    B = 1030
    pre = rng.integers(0, 400, size=B).tolist()
    chunk = rng.integers(1, 4, size=B).tolist()
    wl = WL.extend_workload("band_big_batch", 61, pre, chunk, 16, 2, 300, 16)
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32")
    check(out, oracle_extend(wl), TOL["bf16"], "band, 1030 requests")
    out_bf = run_extend(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


def scale_v_bf16(wl, log2_scale, extremes=False):
    """V rows (pool rows and the new tokens' rows) times 2^log2_scale, which is
    exact in bf16 while no value leaves its normal range.  extremes: dims 0-3 of
    every new V row become +-65280 (the largest bf16 value that f16 holds) and
    +-2^-14 (f16's smallest normal)."""
    def scaled(bits):
        return WL.to_store(codecs.bf16_bits_to_f64(bits) * 2.0 ** log2_scale, "bf16")
    wl.pool_v = WL.SparsePool(*wl.pool_v.shape, "bf16", wl.pool_v.used_rows, scaled(wl.pool_v.values))
    nv = scaled(wl.new_v)
    if extremes:
        nv[..., :4] = WL.to_store(np.array([65280.0, -65280.0, 2.0 ** -14, -(2.0 ** -14)]), "bf16")
    wl.new_v = nv


V_RANGE_SCALES = [(13, True), (-10, False)]  # |v| up to 65280 / about 1e-3 with ~5% f16 subnormals


@pytest.mark.parametrize("window", [128, 1023])
@pytest.mark.parametrize("log2_scale,extremes", V_RANGE_SCALES)
def test_decode_v_range_edges(window, log2_scale, extremes):
    """P.V runs in f16: bf16 V converts exactly up to 65504 and keeps 2^-25
    absolute accuracy below 2^-14.  V at both ends of that range stays within
    the bf16 tolerance, on the window kernel (W = 128, fused store too) and on
    the split-K stream kernel (W = 1023)."""
    say(f"decode V range W={window} scale 2^{log2_scale}")
    wl = WL.decode_workload(f"vrange_{window}", 41 + window, [1, 130, 700, 2000, 3000], 16, 2, window, 16, "bf16",
                            "bf16", with_store=True)
    scale_v_bf16(wl, log2_scale, extremes)
    ref = oracle_decode(wl)
    dw = DeviceWorkload(wl)
    run_store(dw)
    check(run_decode(dw, "f32"), ref, TOL["bf16"], f"decode W={window} V x 2^{log2_scale}")
    if window == 128:
        check(run_decode_store(DeviceWorkload(wl), "f32"), ref, TOL["bf16"], f"fused decode V x 2^{log2_scale}")


@pytest.mark.parametrize("window", [128, 512])
@pytest.mark.parametrize("log2_scale,extremes", V_RANGE_SCALES)
def test_extend_v_range_edges(window, log2_scale, extremes):
    """As test_decode_v_range_edges for extend: the W = 128 ring path and the
    band kernel (W = 512)."""
    say(f"extend V range W={window} scale 2^{log2_scale}")
    wl = WL.extend_workload(f"vrange_{window}", 43 + window, [0, 300, 700], [40, 100, 64], 16, 2, window, 16)
    scale_v_bf16(wl, log2_scale, extremes)
    dw = DeviceWorkload(wl)
    run_store(dw)
    check(run_extend(dw, "f32"), oracle_extend(wl), TOL["bf16"], f"extend W={window} V x 2^{log2_scale}")


def test_extend_bad_qo_indptr_stays_in_bounds():
    """qo_indptr entries outside [0, total_q] or out of order: every request's
    rows are clamped into [0, total_q], so nothing outside `out` is written,
    and swa_validate counts the bad requests exactly as the oracle does."""
    from sliding_window_attention_swa_amd import swa
    wl = WL.extend_workload("badqo", 41, [100, 300, 0], [40, 70, 33], 16, 2, 128, 16)
    say("extend with bad qo_indptr: guard rows around out")
    dw = DeviceWorkload(wl)
    run_store(dw)
    total, B = wl.q.shape[0], wl.batch
    cap = int(wl.seq_lens.astype(np.int64).sum())
    table = torch.empty(cap, dtype=torch.int32, device="cuda")
    indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(dw.index, wl.window, table, indptr, prefix_lens=dw.prefix)
    guard = 64
    want = O.validate(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window, wl.pool_rows,
                      wl.page_size, prefix_lens=wl.prefix_lens, qo_indptr=wl.qo_indptr, total_q=total)
    assert want["qo_bad"] == 0
    for qo in ([-32, 20, 5, total + 50], [total + 5, total + 9, -3, 2], [0, 40, 30, total], [1 << 30, -(1 << 30), 0, 7]):
        big = torch.full((total + 2 * guard, wl.q_heads, wl.head_dim), 7.0, dtype=torch.float32, device="cuda")
        out = big[guard:guard + total]
        qo_t = torch.tensor(qo, dtype=torch.int32, device="cuda")
        swa.swa_extend(dw.q, qo_t, dw.prefix, dw.layer, dw.index, wl.window, out, sinks=dw.sinks, slot_table=table,
                       table_indptr=indptr)
        torch.cuda.synchronize()
        assert bool((big[:guard] == 7.0).all()) and bool((big[guard + total:] == 7.0).all()), qo
        got = swa.swa_validate(dw.index, wl.window, wl.pool_rows, prefix_lens=dw.prefix, qo_indptr=qo_t, total_q=total)
        want = O.validate(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window, wl.pool_rows,
                          wl.page_size, prefix_lens=wl.prefix_lens, qo_indptr=qo, total_q=total)
        assert got == want and got["qo_bad"] > 0, (qo, got, want)


def test_extend_tile_runs_sampled():
    """Enough tiles that every workgroup walks a run of several tiles (band
    blocks rotating through the LDS ring), mixed with band-clipped and
    partial tiles in the same runs."""
    say("extend tile runs (3 requests, 64q/8kv) — sampled rows")
    wl = WL.extend_workload("runs", 77, [300, 129, 16], [1500, 700, 1000], 64, 8, 128, 16, sinks=True)
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32")
    total = wl.q.shape[0]
    rows = np.unique(np.concatenate([np.arange(0, total, 3), np.arange(total - 20, total),
                                     np.arange(1480, 1530), np.arange(2180, 2230)]))
    only = [(int(r), h) for r in rows for h in range(wl.q_heads)]
    check(out, oracle_extend(wl, only=only), TOL["bf16"], "runs sampled")
    out_bf = run_extend(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


def test_extend_c3_full_size_sampled():
    wl = WL.c3_extend_bf16()
    say("extend c3 (4 x (8K prefix + 2K chunk), bf16) — sampled rows")
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32")
    rng = np.random.default_rng(3)
    rows = np.unique(np.concatenate([np.arange(0, 40), np.arange(wl.q.shape[0] - 40, wl.q.shape[0]),
                                     rng.choice(wl.q.shape[0], 300, replace=False)]))
    heads4 = (0, 21, 42, 63)   # one q head of four different kv heads, the first and the last included
    only = {(int(r), h) for r in rows for h in range(wl.q_heads)}
    only |= {(r, h) for r in range(wl.q.shape[0]) for h in heads4}
    ref = oracle_extend(wl, only=sorted(only))
    check(out, ref, TOL["bf16"], "c3: every row x 4 heads, 380 rows x every head")


@pytest.mark.parametrize("window", [512, 4096])
def test_extend_c3_shape_long_window_sampled(window):
    """The C3 shape (4 x (8K prefix + 2K chunk), 64 q / 8 kv heads) with a long
    window, on the band kernel: sampled rows (the first and last of each
    request's chunk and a seeded spread), every q head."""
    wl = WL.c3_extend_bf16(window=window)
    say(f"extend c3 shape, W={window} — sampled rows")
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32")
    rng = np.random.default_rng(window)
    edges = np.concatenate([np.arange(q0, q0 + 3) for q0 in wl.qo_indptr[:-1]] +
                           [np.arange(q1 - 3, q1) for q1 in wl.qo_indptr[1:]])
    rows = np.unique(np.concatenate([edges, rng.choice(wl.q.shape[0], 60, replace=False)]))
    only = [(int(r), h) for r in rows for h in range(wl.q_heads)]
    check(out, oracle_extend(wl, only=only), TOL["bf16"], f"c3 shape W={window} sampled")
    out_bf = run_extend(dw, "bf16")
    assert np.array_equal(device_to_bits(out_bf), bf16_of(out))


# ---------------------------------------------------------------------------
# SWA eviction (mapping maintenance): bit-exact against the oracle
# ---------------------------------------------------------------------------

EVICT_CASES = {
    # name: (lens, page, mode, interval, evicted, protected, live_from)
    "chunk": ([1, 40, 300, 1000, 2049, 129], 16, 0, 0, None, None, None),
    "radix_p64": ([1, 40, 300, 1000, 2049, 129], 64, 1, 0, None, None, None),
    "interval": ([1, 40, 300, 1000, 2049, 129], 16, 0, 128, [0, 0, 96, 800, 1760, 0], None, None),
    "protected": ([1, 40, 300, 1000, 2049, 129], 16, 0, 0, [0, 0, 16, 0, 512, 0], [0, 30, 100, 900, 0, 0], None),
    # stale evicted lengths over spans already tombstoned: only mapped slots are released
    "tombstoned": ([3000, 5000, 700, 4097], 16, 0, 0, None, None, [1000, 4500, 0, 2050]),
    "page1": ([513, 2, 1500], 1, 0, 128, [0, 0, 1000], None, [100, 0, 0]),
    "page3_radix": ([1000, 3001], 3, 1, 0, [7, 0], [0, 10], None),
}


def _evict_gpu(eb, mapping, ev, prot, mode, interval, cap):
    """One swa_evict call on device copies of the batch; returns host copies of
    (mapping, evicted_lens, freed_pages, freed_count)."""
    from sliding_window_attention_swa_amd import swa
    ix = swa.IndexTables(torch.from_numpy(eb.req_to_token).cuda(), torch.from_numpy(eb.req_pool_idx).cuda(),
                         torch.from_numpy(eb.seq_lens).cuda(), None, eb.page_size)
    m = torch.from_numpy(np.array(mapping, dtype=np.int64)).cuda()
    evd = torch.from_numpy(np.asarray(ev, dtype=np.int32)).cuda()
    pages = torch.full((max(cap, 1),), -9, dtype=torch.int64, device="cuda")
    count = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    prot_d = None if prot is None else torch.from_numpy(np.asarray(prot, np.int32)).cuda()
    swa.swa_evict(ix, m, torch.from_numpy(eb.pre_lens).cuda(), evd, eb.window, pages[:cap] if cap else pages[:0],
                  count, mode=mode, interval=interval, protected_lens=prot_d)
    torch.cuda.synchronize()
    return m.cpu().numpy(), evd.cpu().numpy(), pages.cpu().numpy()[:cap], int(count.item())


def _check_evict(eb, ev, prot, mode, interval):
    want_m, want_ev, want_pages = O.evict(eb.req_to_token, eb.req_pool_idx, eb.full_to_swa, eb.pre_lens, ev,
                                          eb.window, eb.page_size, mode=mode, interval=interval,
                                          protected_lens=prot)
    assert want_pages.size > 0
    m, evd, pages, count = _evict_gpu(eb, eb.full_to_swa, ev, prot, mode, interval, want_pages.size + 5)
    assert np.array_equal(m, want_m)
    assert np.array_equal(evd, want_ev)
    assert count == want_pages.size
    assert np.array_equal(pages[:count], want_pages) and np.all(pages[count:] == -9)
    return m, evd, want_m, want_pages


@pytest.mark.parametrize("name", list(EVICT_CASES))
def test_evict_bit_exact(name):
    lens, P, mode, interval, ev, prot, live = EVICT_CASES[name]
    say(f"evict {name}")
    eb = WL.evict_batch("ev" + name, 41, lens, P, 128, live_from=live)
    ev = np.zeros(len(lens), np.int32) if ev is None else np.asarray(ev, np.int32)
    m, evd, want_m, want_pages = _check_evict(eb, ev, prot, mode, interval)
    # releasing again frees nothing and changes nothing
    m2, evd2, pages2, count2 = _evict_gpu(eb, m, evd, prot, mode, interval, 4)
    assert count2 == 0 and np.array_equal(m2, m) and np.array_equal(evd2, evd) and np.all(pages2 == -9)
    # a short page buffer: its prefix is written, the count is the full number
    m3, _, pages3, count3 = _evict_gpu(eb, eb.full_to_swa, ev, prot, mode, interval, 3)
    assert count3 == want_pages.size and np.array_equal(pages3, want_pages[:3]) and np.array_equal(m3, want_m)
    # no page buffer at all
    _, _, _, count4 = _evict_gpu(eb, eb.full_to_swa, ev, prot, mode, interval, 0)
    assert count4 == want_pages.size


def test_evict_empty_batch():
    from sliding_window_attention_swa_amd import swa
    say("evict empty batch")
    r2t = torch.zeros((1, 16), dtype=torch.int32, device="cuda")
    e = torch.zeros(0, dtype=torch.int32, device="cuda")
    ix = swa.IndexTables(r2t, e, e, None, 16)
    m = torch.tensor([0, 5, -1], dtype=torch.int64, device="cuda")
    count = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    swa.swa_evict(ix, m, e, e, 128, torch.empty(0, dtype=torch.int64, device="cuda"), count)
    torch.cuda.synchronize()
    assert int(count.item()) == 0 and m.tolist() == [0, 5, -1]


def test_evict_after_prefill_full_size():
    """The benchmark's eviction batch at its full size (B = 256, lognormal
    lengths up to 64K, P = 64, decode interval 128), compared in full."""
    say("evict after prefill, full size")
    eb = WL.evict_after_prefill()
    _check_evict(eb, eb.evicted_lens, None, 0, 128)


def test_evict_then_decode_unchanged():
    """Releasing everything left of the current token's window changes neither
    the window tables nor the decode output, bit for bit."""
    wl = WL.decode_workload("evdec", 43, [1, 40, 300, 1000, 129, 4000], 16, 2, 128, 16, "bf16", "bf16",
                            sinks=True, live_margin=100000)
    dw = DeviceWorkload(wl)
    say("evict then decode")
    before = run_decode(dw, "f32").cpu().numpy()
    eb = WL.EvictBatch("evdec", wl.batch, 16, 128, wl.seq_lens, (wl.seq_lens - 1).astype(np.int32),
                       np.zeros(wl.batch, np.int32), wl.req_to_token, wl.req_pool_idx, wl.full_to_swa, wl.n_full,
                       wl.n_swa)
    m, _, _, count = _evict_gpu(eb, wl.full_to_swa, eb.evicted_lens, None, 0, 0, 4096)
    assert count > 0 and np.count_nonzero(m == 0) > np.count_nonzero(wl.full_to_swa == 0)
    dw.map.copy_(torch.from_numpy(m).cuda())
    after = run_decode(dw, "f32").cpu().numpy()
    assert np.array_equal(before, after)


# ---------------------------------------------------------------------------
# paired allocation: bit-exact against the oracle
# ---------------------------------------------------------------------------

ALLOC_CASES = {
    # name: (pre_lens, seq_lens, page)
    "mixed_p16": ([0, 5, 16, 31, 100, 0, 700, 17], [40, 16, 17, 64, 100, 1, 3000, 4113], 16),
    "p1": ([0, 3, 9, 50], [7, 3, 300, 51], 1),
    "p64_chunks": ([8192, 8000, 8191, 1], [10240, 10048, 10239, 2049], 64),
    "p3_ragged": ([2, 0, 11], [2000, 5, 12], 3),
}


def _alloc_gpu(ab, decode, two_pools=True, host_lens=True, with_swa_out=True, free_full=None, free_swa=None):
    from sliding_window_attention_swa_amd import swa
    dev = lambda a: torch.from_numpy(np.ascontiguousarray(a)).cuda()
    n = ab.batch if decode else int((ab.seq_lens.astype(np.int64) - ab.pre_lens).sum())
    out_full = torch.full((max(n, 1),), -9, dtype=torch.int64, device="cuda")[:n]
    out_swa = torch.full((max(n, 1),), -9, dtype=torch.int64, device="cuda")[:n] if with_swa_out else None
    new_pages = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    m = dev(ab.full_to_swa) if two_pools else None
    ff = dev(ab.free_full if free_full is None else free_full)
    fs = dev(ab.free_swa if free_swa is None else free_swa) if two_pools else None
    if decode:
        ok = swa.swa_alloc_decode(dev(ab.seq_lens), dev(ab.last_loc), ab.page_size, ff, out_full, free_swa=fs,
                                  full_to_swa=m, out_swa=out_swa, new_pages=new_pages,
                                  seq_lens_host=ab.seq_lens if host_lens else None)
    else:
        ok = swa.swa_alloc_extend(dev(ab.pre_lens), dev(ab.seq_lens), dev(ab.last_loc), ab.page_size, ff, out_full,
                                  free_swa=fs, full_to_swa=m, out_swa=out_swa, new_pages=new_pages,
                                  pre_lens_host=ab.pre_lens if host_lens else None,
                                  seq_lens_host=ab.seq_lens if host_lens else None)
    torch.cuda.synchronize()
    return (ok, out_full.cpu().numpy(), None if out_swa is None else out_swa.cpu().numpy(),
            None if m is None else m.cpu().numpy(), int(new_pages.item()))


def _check_alloc(ab, decode, two_pools=True, with_swa_out=True):
    want = O.alloc_paired(ab.pre_lens, ab.seq_lens, ab.last_loc, ab.free_full, ab.free_swa if two_pools else None,
                          ab.full_to_swa, ab.page_size, decode=decode)
    assert want is not None
    ok, full, swa_out, m, pages = _alloc_gpu(ab, decode, two_pools, with_swa_out=with_swa_out)
    assert ok
    assert np.array_equal(full, want[0])
    assert pages == want[3]
    if two_pools:
        assert np.array_equal(m, want[2])
        if with_swa_out:
            assert np.array_equal(swa_out, want[1])
    return want


@pytest.mark.parametrize("name", list(ALLOC_CASES))
@pytest.mark.parametrize("two_pools", [True, False])
def test_alloc_extend_bit_exact(name, two_pools):
    pre, seq, P = ALLOC_CASES[name]
    say(f"alloc_extend {name} two_pools={two_pools}")
    ab = WL.alloc_batch("al" + name, 51, pre, seq, P)
    _check_alloc(ab, decode=False, two_pools=two_pools)


@pytest.mark.parametrize("P", [1, 16, 64])
def test_alloc_decode_bit_exact(P):
    say(f"alloc_decode P={P}")
    rng = np.random.default_rng(60 + P)
    pre = rng.integers(1, 3 * P + 40, 300)   # 300 requests: two workgroups
    pre[:6] = [P, 2 * P, 1, P - 1 if P > 1 else 1, 5 * P, 7]
    ab = WL.alloc_batch(f"ald{P}", 52, pre, pre + 1, P)
    want = _check_alloc(ab, decode=True)
    assert want[3] == int(np.sum(pre % P == 0))
    _check_alloc(ab, decode=True, with_swa_out=False)


def test_alloc_prefill_chunk_full_size():
    """The benchmark's extend allocation: 256 requests of lognormal length take
    a 2048-position chunk each (P = 64); the bound cannot prove the fit, the
    exact count from the host lengths can."""
    say("alloc prefill chunk, full size")
    ab = WL.alloc_prefill_chunk()
    _check_alloc(ab, decode=False)


def test_alloc_decode_step_full_size():
    say("alloc decode step, full size")
    _check_alloc(WL.alloc_decode_step(), decode=True)


def test_alloc_no_space_changes_nothing():
    say("alloc no space")
    ab = WL.alloc_batch("alns", 53, [0, 20, 64], [100, 84, 130], 16)
    need = O.pages_needed(ab.pre_lens, ab.seq_lens, 16)
    # one page short on the SWA list: not allocated, outputs and mapping untouched
    ok, full, swa_out, m, pages = _alloc_gpu(ab, False, free_swa=ab.free_swa[:need - 1])
    assert not ok and np.all(full == -9) and np.all(swa_out == -9) and pages == -9
    assert np.array_equal(m, ab.full_to_swa)
    # exactly enough (16 pages), proven only by the exact count: the bound is 230 // 16 + 3 + 1 = 18
    want = O.alloc_paired(ab.pre_lens, ab.seq_lens, ab.last_loc, ab.free_full[:need], ab.free_swa[:need],
                          ab.full_to_swa, 16)
    ok, full, swa_out, m, pages = _alloc_gpu(ab, False, free_full=ab.free_full[:need], free_swa=ab.free_swa[:need])
    assert ok and np.array_equal(full, want[0]) and np.array_equal(swa_out, want[1]) and np.array_equal(m, want[2])
    # without host lengths the same call cannot be proven and is refused
    ok, *_ = _alloc_gpu(ab, False, host_lens=False, free_full=ab.free_full[:need], free_swa=ab.free_swa[:need])
    assert not ok


def test_alloc_empty_batch():
    from sliding_window_attention_swa_amd import swa
    say("alloc empty batch")
    e32 = torch.zeros(0, dtype=torch.int32, device="cuda")
    e64 = torch.zeros(0, dtype=torch.int64, device="cuda")
    pages = torch.full((1,), -9, dtype=torch.int64, device="cuda")
    free = torch.arange(1, 5, dtype=torch.int64, device="cuda")
    assert swa.swa_alloc_extend(e32, e32, e64, 16, free, e64, new_pages=pages)
    torch.cuda.synchronize()
    assert int(pages.item()) == 0


def test_alloc_then_translate_and_window():
    """The allocation's mapping is the one the path reads: translate_loc of the
    new full slots gives the new SWA slots, and after writing the new positions
    into req_to_token the window tables of the grown requests hold them."""
    from sliding_window_attention_swa_amd import swa
    say("alloc then translate")
    ab = WL.alloc_batch("alrt", 54, [0, 5, 300, 1000], [200, 6, 301, 1100], 16)
    ok, full, swa_out, m, _ = _alloc_gpu(ab, False)
    assert ok
    loc = torch.empty(full.size, dtype=torch.int64, device="cuda")
    swa.swa_translate_loc(torch.from_numpy(full).cuda(), torch.from_numpy(m).cuda(), loc)
    torch.cuda.synchronize()
    assert np.array_equal(loc.cpu().numpy(), swa_out)
    r2t = ab.req_to_token.copy()
    at = 0
    for b in range(ab.batch):
        n = int(ab.seq_lens[b] - ab.pre_lens[b])
        r2t[ab.req_pool_idx[b], ab.pre_lens[b]:ab.seq_lens[b]] = full[at:at + n]
        at += n
    want = O.window_table(r2t, ab.req_pool_idx, ab.seq_lens, m, 128)
    ix = swa.IndexTables(torch.from_numpy(r2t).cuda(), torch.from_numpy(ab.req_pool_idx).cuda(),
                         torch.from_numpy(ab.seq_lens).cuda(), torch.from_numpy(m).cuda(), 16)
    table = torch.empty(ab.batch * 129, dtype=torch.int32, device="cuda")
    indptr = torch.empty(ab.batch + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(ix, 128, table, indptr)
    torch.cuda.synchronize()
    got_ptr = indptr.cpu().numpy()
    assert np.array_equal(got_ptr, want[1])
    assert np.array_equal(table.cpu().numpy()[:got_ptr[-1]], want[0])
    assert np.all(want[0] > 0)   # every slot of the grown windows is live


# ---------------------------------------------------------------------------
# unified pool: same kernels over dense per-layer views of one raw buffer
# ---------------------------------------------------------------------------

NAN_BF16 = np.uint16(0x7FC0)


def _unified_raw(ub, anchor=256):
    """The raw byte buffer of a unified batch: NaN everywhere (so stray reads
    show), each live token's rows placed by the oracle's envelope formula."""
    itemsize = 2
    g = O.unified_geometry(ub.layers, ub.kv_heads, ub.head_dim, itemsize, ub.page_size, ub.n_phys)
    raw = np.empty(anchor + g["total_bytes"] + g["tail_pad"], dtype=np.uint8)
    raw.view(np.uint16)[:] = NAN_BF16
    P = ub.page_size
    for i, t in enumerate(ub.live_tokens):
        page, off = int(ub.v2p[t // P]), int(t % P)
        for layer in range(ub.layers):
            for kv, rows in ((0, ub.k_rows), (1, ub.v_rows)):
                at = O.envelope_offset(anchor, page, layer, kv, off, ub.layers, g["row_bytes"], P)
                raw[at:at + g["row_bytes"]] = rows[layer, i].reshape(-1).view(np.uint8)
    return raw, g


def test_unified_kernel_ids_bit_exact():
    from sliding_window_attention_swa_amd import swa
    say("unified kernel ids")
    ub = WL.unified_batch("uk", 61, [1, 40, 300, 1000, 129], 3, 8, 2, 128, 16, with_rows=False)
    virt = np.arange(ub.v2p.size * ub.page_size, dtype=np.int64)
    want = O.unified_kernel_ids(virt, ub.v2p, ub.page_size, 2 * ub.layers)
    out = torch.empty(virt.size, dtype=torch.int64, device="cuda")
    d_virt = torch.from_numpy(virt).cuda()
    swa.swa_translate_kernel_ids(d_virt, torch.from_numpy(ub.v2p).cuda(), ub.page_size, 2 * ub.layers, out)
    # in place, and ids outside the page table (negative, past the last page) read the sink row 0
    odd = torch.tensor([-1, -100, virt.size, virt.size + 17, 5], dtype=torch.int64, device="cuda")
    swa.swa_translate_kernel_ids(odd, torch.from_numpy(ub.v2p).cuda(), ub.page_size, 2 * ub.layers, odd)
    torch.cuda.synchronize()
    assert np.array_equal(out.cpu().numpy(), want)
    assert odd.cpu().tolist() == [0, 0, 0, 0, int(want[5])]


@pytest.mark.parametrize("P", [1, 16, 64])
def test_unified_window_table_bit_exact(P):
    from sliding_window_attention_swa_amd import swa
    say(f"unified window table P={P}")
    ub = WL.unified_batch(f"uw{P}", 62, [1, 40, 300, 1000, 129, 4000], 4, 8, 2, 128, P, with_rows=False)
    mult = 2 * ub.layers
    want = O.window_table(ub.req_to_token, ub.req_pool_idx, ub.seq_lens, O.unified_mapping(ub.v2p, P, mult), 128)
    ix = swa.IndexTables(torch.from_numpy(ub.req_to_token).cuda(), torch.from_numpy(ub.req_pool_idx).cuda(),
                         torch.from_numpy(ub.seq_lens).cuda(), None, P)
    table = torch.empty(int(want[1][-1]) + 7, dtype=torch.int32, device="cuda")
    indptr = torch.empty(ub.batch + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window_unified(ix, torch.from_numpy(ub.v2p).cuda(), mult, 128, table, indptr)
    torch.cuda.synchronize()
    assert np.array_equal(indptr.cpu().numpy(), want[1])
    assert np.array_equal(table.cpu().numpy()[:want[1][-1]], want[0])


def test_unified_store_places_rows_byte_exact():
    """kv_store through the library's views at kernel-facing ids writes each
    row exactly where the oracle's envelope formula puts it."""
    from sliding_window_attention_swa_amd import swa
    say("unified store")
    ub = WL.unified_batch("us", 63, [40, 300, 129, 17], 3, 8, 2, 128, 16, with_rows=False)
    anchor = 512
    g = O.unified_geometry(ub.layers, ub.kv_heads, ub.head_dim, 2, 16, ub.n_phys)
    raw = torch.zeros(anchor + g["total_bytes"] + g["tail_pad"], dtype=torch.uint8, device="cuda")
    views = swa.swa_unified_layer_views(raw, anchor, ub.layers, ub.kv_heads, ub.head_dim, torch.bfloat16, 16,
                                        ub.n_phys)
    virt = ub.req_to_token[ub.req_pool_idx, ub.seq_lens - 1].astype(np.int64)   # each request's current token
    ids = torch.empty(ub.batch, dtype=torch.int64, device="cuda")
    swa.swa_translate_kernel_ids(torch.from_numpy(virt).cuda(), torch.from_numpy(ub.v2p).cuda(), 16, 2 * ub.layers,
                                 ids)
    for layer in range(ub.layers):
        swa.swa_kv_store(views[layer], ids, bits_to_device(ub.new_k[layer], "bf16"),
                         bits_to_device(ub.new_v[layer], "bf16"))
    torch.cuda.synchronize()
    want = np.zeros(raw.numel(), dtype=np.uint8)
    for b, t in enumerate(virt):
        page, off = int(ub.v2p[t // 16]), int(t % 16)
        for layer in range(ub.layers):
            for kv, rows in ((0, ub.new_k), (1, ub.new_v)):
                at = O.envelope_offset(anchor, page, layer, kv, off, ub.layers, g["row_bytes"], 16)
                want[at:at + g["row_bytes"]] = rows[layer, b].reshape(-1).view(np.uint8)
    assert np.array_equal(raw.cpu().numpy(), want)


@pytest.mark.parametrize("P", [16, 64])
def test_unified_decode_matches_oracle_and_two_pool(P):
    from sliding_window_attention_swa_amd import swa
    say(f"unified decode P={P}")
    ub = WL.unified_batch(f"ud{P}", 64, [1, 40, 300, 1000, 129, 2049], 3, 16, 2, 128, P)
    mult = 2 * ub.layers
    raw_h, g = _unified_raw(ub)
    raw = torch.from_numpy(raw_h).cuda()
    views = swa.swa_unified_layer_views(raw, 256, ub.layers, ub.kv_heads, ub.head_dim, torch.bfloat16, P, ub.n_phys)
    ks, vs = O.unified_views(raw_h, 256, ub.layers, ub.kv_heads, ub.head_dim, np.uint16, P, ub.n_phys)
    m_unified = O.unified_mapping(ub.v2p, P, mult)
    d_r2t = torch.from_numpy(ub.req_to_token).cuda()
    d_rows = torch.from_numpy(ub.req_pool_idx).cuda()
    d_lens = torch.from_numpy(ub.seq_lens).cuda()
    ix = swa.IndexTables(d_r2t, d_rows, d_lens, None, P)
    cap = ub.batch * 129
    table = torch.empty(cap, dtype=torch.int32, device="cuda")
    indptr = torch.empty(ub.batch + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window_unified(ix, torch.from_numpy(ub.v2p).cuda(), mult, 128, table, indptr)
    q = bits_to_device(ub.q, "bf16")
    sinks = torch.from_numpy(ub.sinks).cuda()
    # the two-pool form of the same data: pool row s = virtual id s (identity mapping, tombstones 0)
    kid = m_unified[:-1]
    ident = np.where(kid > 0, np.arange(kid.size), 0).astype(np.int64)
    ident = np.concatenate([ident, [-1]])
    ix2 = swa.IndexTables(d_r2t, d_rows, d_lens, torch.from_numpy(ident).cuda(), P)
    table2 = torch.empty(cap, dtype=torch.int32, device="cuda")
    indptr2 = torch.empty(ub.batch + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(ix2, 128, table2, indptr2)
    for layer in range(ub.layers):
        out = torch.empty((ub.batch, ub.q_heads, ub.head_dim), dtype=torch.float32, device="cuda")
        swa.swa_decode(q, views[layer], ix, 128, out, sinks=sinks, slot_table=table, table_indptr=indptr,
                       num_splits=1, use_map=False)
        pool_k = bits_to_device(np.asarray(ks[layer])[kid], "bf16")
        pool_v = bits_to_device(np.asarray(vs[layer])[kid], "bf16")
        out2 = torch.empty_like(out)
        swa.swa_decode(q, swa.KvLayer(pool_k, pool_v), ix2, 128, out2, sinks=sinks, slot_table=table2,
                       table_indptr=indptr2, num_splits=1)
        torch.cuda.synchronize()
        want = O.decode(ub.q, "bf16", ks[layer], vs[layer], "bf16", ub.req_to_token, ub.req_pool_idx, ub.seq_lens,
                        m_unified, 128, ub.sinks)
        check(out, want, TOL["bf16"], f"unified decode layer {layer}")
        assert torch.equal(out, out2)


# ---------------------------------------------------------------------------
# attention variants: single-pool windowed mode, chunked local attention,
# per-request SWA ring
# ---------------------------------------------------------------------------

@pytest.mark.parametrize("G,W,P", [(8, 128, 16), (1, 20, 1), (16, 300, 64)])
def test_single_pool_windowed_decode(G, W, P):
    say(f"single-pool decode G={G} W={W} P={P}")
    wl = WL.decode_workload(f"sp{G}_{W}", 81, [1, 40, 300, 1000, 129, 2000], 2 * G, 2, W, P, "bf16", "bf16",
                            with_store=True, two_pools=False)
    assert wl.full_to_swa is None
    dw = DeviceWorkload(wl)
    run_store(dw)
    splits = None if W <= 255 else 3
    check(run_decode(dw, "f32", num_splits=splits), oracle_decode(wl), TOL["bf16"], "single-pool decode")


def test_single_pool_windowed_extend():
    say("single-pool extend")
    wl = WL.extend_workload("spx", 82, [0, 100, 700], [300, 33, 129], 16, 2, 128, 16, two_pools=False)
    dw = DeviceWorkload(wl)
    run_store(dw)
    check(run_extend(dw, "f32"), oracle_extend(wl), TOL["bf16"], "single-pool extend")


@pytest.mark.parametrize("C,W", [(64, -1), (256, -1), (1000, -1), (100, 128), (1, -1)])
def test_chunked_local_decode(C, W):
    """Chunked local decode is swa_decode over the chunked window table."""
    from sliding_window_attention_swa_amd import swa
    say(f"chunked decode C={C} W={W}")
    lens = [1, 40, 256, 257, 1000, 1001, 2048, 2100]
    wl = WL.decode_workload(f"ch{C}_{W}", 83, lens, 16, 2, W, 16, "bf16", "bf16", two_pools=False)
    dw = DeviceWorkload(wl)
    B = wl.batch
    table = torch.empty(B * min(C, 2100), dtype=torch.int32, device="cuda")
    indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window_chunked(dw.index, W, C, table, indptr, use_map=False)
    want_t = O.window_table(wl.req_to_token, wl.req_pool_idx, wl.seq_lens, None, W, chunk=C)
    torch.cuda.synchronize()
    assert np.array_equal(indptr.cpu().numpy(), want_t[1])
    assert np.array_equal(table.cpu().numpy()[:want_t[1][-1]], want_t[0])
    keys = min(C, W + 1) if W >= 0 else C
    if keys <= 256:
        win, splits, ws = keys - 1, 1, None
    else:
        win = -1
        splits, ws_bytes = swa.swa_decode_plan(B, wl.q_heads, wl.kv_heads, wl.head_dim, -1, keys)
        ws = torch.empty(max(ws_bytes // 4, 1), dtype=torch.float32, device="cuda")
    out = torch.empty((B, wl.q_heads, wl.head_dim), dtype=torch.float32, device="cuda")
    swa.swa_decode(dw.q, dw.layer, dw.index, win, out, sinks=dw.sinks, slot_table=table, table_indptr=indptr,
                   num_splits=splits, workspace=ws, use_map=False)
    torch.cuda.synchronize()
    check(out, oracle_decode(wl, chunk=C), TOL["bf16"], f"chunked decode C={C}")


CHUNKED_EXTEND = [
    # (G, W, C, prefix_lens, chunk_lens)
    (8, -1, 16, [0, 100, 37], [300, 33, 129]),
    (8, -1, 100, [0, 250, 1000], [700, 129, 64]),
    (8, 128, 48, [0, 300], [400, 77]),
    (1, -1, 64, [10, 0], [200, 150]),
    (16, -1, 80, [0, 90], [260, 70]),
    (8, -1, 4096, [0, 4000], [1100, 300]),
]


@pytest.mark.parametrize("case", range(len(CHUNKED_EXTEND)))
def test_chunked_local_extend(case):
    G, W, C, pre, new = CHUNKED_EXTEND[case]
    say(f"chunked extend G={G} W={W} C={C}")
    wl = WL.extend_workload(f"chx{case}", 84 + case, pre, new, 2 * G, 2, W, 16, two_pools=False)
    dw = DeviceWorkload(wl)
    run_store(dw)
    out = run_extend(dw, "f32", chunk=C)
    check(out, oracle_extend(wl, chunk=C), TOL["bf16"], f"chunked extend C={C}")
    bf = run_extend(dw, "bf16", chunk=C)
    assert np.array_equal(bf16_of(out), device_to_bits(bf))


def _ring_pool(rb, R):
    """The ring pool of a ring batch: every live position's rows at its ring row
    (placed with the oracle's ring_slot), NaN elsewhere."""
    rows = rb.request_slots * R
    pk = np.full((rows, rb.kv_heads, rb.head_dim), NAN_BF16, dtype=np.uint16)
    pv = pk.copy()
    for b in range(rb.batch):
        for n, j in enumerate(range(int(rb.live_lo[b]), int(rb.prefix_lens[b]))):
            s = O.ring_slot(int(rb.req_pool_idx[b]), j, R)
            pk[s] = rb.k_rows[b][n]
            pv[s] = rb.v_rows[b][n]
    return pk, pv


@pytest.mark.parametrize("decode,W,ring,P", [(True, 128, 129, 16), (True, 20, 21, 1), (False, 128, 128 + 300, 64),
                                             (False, 32, 40, 16)])
def test_ring_attention(decode, W, ring, P):
    """Per-request SWA ring: ring locations and the window table are bit-exact,
    the new rows land in the ring, and attention matches the oracle over the
    same ring layout."""
    from sliding_window_attention_swa_amd import swa
    say(f"ring decode={decode} W={W} ring={ring} P={P}")
    if decode:
        rb = WL.ring_batch(f"rd{W}", 91, [0, 5, 300, 1000, 128, 129], [1] * 6, 16, 2, W)
    else:
        # each request's step spans min(prefix, W) + (ring - W) <= ring positions: no wrap
        rb = WL.ring_batch(f"rx{W}", 92, [0, 40, 700], [ring - W] * 3, 16, 2, W)
    R = O.ring_rows(ring, P)
    B, total = rb.batch, int((rb.seq_lens - rb.prefix_lens).sum())
    pk, pv = _ring_pool(rb, R)
    d_rows = torch.from_numpy(rb.req_pool_idx).cuda()
    d_lens = torch.from_numpy(rb.seq_lens).cuda()
    d_pre = torch.from_numpy(rb.prefix_lens).cuda()
    stride = int(rb.seq_lens.max())
    # where the new positions go
    locs = torch.empty(total, dtype=torch.int64, device="cuda")
    swa.swa_ring_locs(d_rows, d_lens, rb.request_slots, R, locs, prefix_lens=None if decode else d_pre)
    want_locs = np.concatenate([[O.ring_slot(int(rb.req_pool_idx[b]), j, R)
                                 for j in range(int(rb.prefix_lens[b]), int(rb.seq_lens[b]))] for b in range(B)])
    # the window table
    ring_r2t = O.ring_req_to_token(rb.request_slots, stride, R)
    want_t = O.window_table(ring_r2t, rb.req_pool_idx, rb.seq_lens, None, W,
                            prefix_lens=None if decode else rb.prefix_lens)
    table = torch.empty(int(want_t[1][-1]) + 5, dtype=torch.int32, device="cuda")
    indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window_ring(d_rows, d_lens, rb.request_slots, stride, R, W, table, indptr,
                                  prefix_lens=None if decode else d_pre)
    torch.cuda.synchronize()
    assert np.array_equal(locs.cpu().numpy(), want_locs)
    assert np.array_equal(indptr.cpu().numpy(), want_t[1])
    assert np.array_equal(table.cpu().numpy()[:want_t[1][-1]], want_t[0])
    # store the new rows through the ring, then attend
    k = bits_to_device(pk, "bf16")
    v = bits_to_device(pv, "bf16")
    layer = swa.KvLayer(k, v)
    swa.swa_kv_store(layer, locs, bits_to_device(rb.new_k, "bf16"), bits_to_device(rb.new_v, "bf16"))
    pk2, pv2 = O.kv_store(pk, pv, want_locs, rb.new_k, rb.new_v, "bf16", "bf16")
    torch.cuda.synchronize()
    assert np.array_equal(device_to_bits(k), pk2) and np.array_equal(device_to_bits(v), pv2)
    ix = swa.IndexTables(torch.from_numpy(ring_r2t.astype(np.int32)).cuda(), d_rows, d_lens, None, P)
    q = bits_to_device(rb.q, "bf16")
    sinks = torch.from_numpy(rb.sinks).cuda()
    out = torch.empty((total, rb.q_heads, rb.head_dim), dtype=torch.float32, device="cuda")
    if decode:
        swa.swa_decode(q, layer, ix, W, out, sinks=sinks, slot_table=table, table_indptr=indptr, use_map=False)
        want = O.decode(rb.q, "bf16", pk2, pv2, "bf16", ring_r2t, rb.req_pool_idx, rb.seq_lens, None, W, rb.sinks)
    else:
        qo = np.concatenate([[0], np.cumsum(rb.seq_lens - rb.prefix_lens)]).astype(np.int32)
        swa.swa_extend(q, torch.from_numpy(qo).cuda(), d_pre, layer, ix, W, out, sinks=sinks, slot_table=table,
                       table_indptr=indptr, use_map=False)
        want = O.extend(rb.q, "bf16", qo, rb.prefix_lens, pk2, pv2, "bf16", ring_r2t, rb.req_pool_idx, rb.seq_lens,
                        None, W, rb.sinks)
    torch.cuda.synchronize()
    check(out, want, TOL["bf16"], "ring attention")
