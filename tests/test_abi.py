"""C-ABI checks that need no GPU: the library loads, exports every symbol the
header declares, and rejects bad arguments on the host before any launch."""

import ctypes
import os
import re

import numpy as np
import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADERS = [os.path.join(ROOT, "include", h) for h in ("swa.h", "swa_probe.h")]


@pytest.fixture(scope="module")
def swa():
    from sliding_window_attention_swa_amd import swa as mod
    return mod


def declared_functions():
    names = set()
    for h in HEADERS:
        text = re.sub(r"/\*.*?\*/", "", open(h).read(), flags=re.S)
        names |= set(re.findall(r"\b(swa_[a-z_]+)\s*\(", text))
    return sorted(names)


def test_every_header_is_checked():
    assert sorted(os.listdir(os.path.join(ROOT, "include"))) == sorted(os.path.basename(h) for h in HEADERS)


def test_header_symbols_exported(swa):
    names = declared_functions()
    assert len(names) >= 8
    for n in names:
        assert hasattr(swa.lib, n), f"{n} declared in include/ but not exported"
    assert set(names) == set(swa.EXPORTS)


def test_status_strings(swa):
    for code in (0, -1, -2, -3, -4, -5, -6):
        assert swa.status_string(code) not in ("", "unknown status")
    assert swa.status_string(-99) == "unknown status"


def test_pool_config_matches_cell_formula(swa):
    from oracle import swa_oracle as O
    for avail, ratio, P, W, Lf, F, Ls, S in [(36_077_256_295, 0.1, 64, 128, 9, 2048, 39, 4096),
                                             (10 ** 11, 0.8, 16, 128, 9, 1000, 39, 2000),
                                             (10 ** 10, 0.05, 1, 128, 9, 1000, 39, 2000),
                                             (5 * 10 ** 9, 0.3, 64, 4095, 0, 0, 10, 4096)]:
        st, nf, ns = swa.swa_pool_config(avail, ratio, P, W, Lf, F, Ls, S)
        _, onf, ons = O.pool_config(avail, ratio, P, W, Lf, F, Ls, S)
        assert st == 0 and (nf, ns) == (onf, ons)
    st, nf, ns = swa.swa_pool_config(192 * 4096 * 10, 0.01, 64, 128, 0, 0, 10, 4096)
    assert st == swa.SWA_E_NOSPACE
    with pytest.raises(swa.SwaError):
        swa.swa_pool_config(10 ** 9, 0.5, 0, 128, 9, 1000, 39, 2000)  # page_size 0
    with pytest.raises(swa.SwaError):
        swa.swa_pool_config(10 ** 9, -0.5, 64, 128, 9, 1000, 39, 2000)


def test_decode_plan(swa):
    ns, ws = swa.swa_decode_plan(64, 64, 8, 128, 128, 8192)
    assert ns == 1 and ws == 0  # SWA layers: one split, no workspace
    ns, ws = swa.swa_decode_plan(32, 64, 4, 128, -1, 32768)
    assert ns > 1 and ws == 32 * 64 * ns * (2 + 128) * 4
    ns, _ = swa.swa_decode_plan(1, 8, 8, 128, -1, 100)
    assert ns == 1
    with pytest.raises(swa.SwaError) as e:
        swa.swa_decode_plan(4, 64, 8, 64, 128, 100)
    assert e.value.status == swa.SWA_E_SHAPE
    with pytest.raises(swa.SwaError) as e:
        swa.swa_decode_plan(4, 24, 8, 128, 128, 100)  # group 3
    assert e.value.status == swa.SWA_E_SHAPE


FAKE = 0x10000  # a 16-byte aligned non-null address that is never dereferenced


def layer(swa, dtype=1, head_dim=128, kv_heads=8, rows=1024, k=FAKE, v=FAKE, scale=1.0):
    return swa.KvLayerStruct(k, v, rows, kv_heads, head_dim, dtype, scale, scale)


def index(swa, batch=2, map_ptr=FAKE):
    return swa.IndexStruct(FAKE, 3, 100, FAKE, FAKE, map_ptr, 50 if map_ptr else 0, batch, 16)


def decode(swa, ly, ix, q_dtype=1, q_heads=64, out_dtype=0, splits=1, ws=None, ws_bytes=0, window=128,
           table=FAKE, indptr=FAKE, q=FAKE, out=FAKE, scale=0.088):
    return swa.lib.swa_decode(q, q_dtype, q_heads, ctypes.byref(ly), ctypes.byref(ix), table, indptr, 1000, window,
                              None, scale, out, out_dtype, splits, ws, ws_bytes, None)


def test_decode_argument_errors(swa):
    E = swa
    ly, ix = layer(swa), index(swa)
    assert decode(swa, layer(swa, head_dim=64), ix) == E.SWA_E_SHAPE
    assert decode(swa, ly, ix, q_heads=24) == E.SWA_E_SHAPE
    assert decode(swa, ly, ix, q_heads=64 * 4) == E.SWA_E_SHAPE  # group 32
    assert decode(swa, ly, ix, q_dtype=0) == E.SWA_E_DTYPE        # f32 q with bf16 K/V
    assert decode(swa, layer(swa, dtype=0), ix, q_dtype=1) == E.SWA_E_DTYPE
    assert decode(swa, ly, ix, out_dtype=2) == E.SWA_E_DTYPE
    assert decode(swa, layer(swa, dtype=7), ix) == E.SWA_E_DTYPE
    assert decode(swa, ly, ix, q=None) == E.SWA_E_ARG
    assert decode(swa, ly, ix, out=FAKE + 4) == E.SWA_E_ARG        # misaligned
    assert decode(swa, ly, ix, window=-2) == E.SWA_E_ARG
    assert decode(swa, ly, ix, splits=0) == E.SWA_E_ARG
    assert decode(swa, ly, ix, splits=4) == E.SWA_E_WORKSPACE
    assert decode(swa, ly, ix, splits=4, ws=FAKE, ws_bytes=100) == E.SWA_E_WORKSPACE
    assert decode(swa, ly, ix, table=None) == E.SWA_E_ARG          # indptr without table
    assert decode(swa, layer(swa, k=None), ix) == E.SWA_E_ARG
    assert decode(swa, layer(swa, rows=0), ix) == E.SWA_E_ARG
    assert decode(swa, layer(swa, dtype=2, scale=0.0), ix) == E.SWA_E_ARG  # fp8 scale must be > 0
    assert decode(swa, layer(swa, rows=1 << 31), ix) == E.SWA_E_SHAPE       # slots must fit int32
    bad_ix = swa.IndexStruct(FAKE, 3, 100, FAKE, None, FAKE, 50, 2, 16)     # no seq_lens
    assert decode(swa, ly, bad_ix) == E.SWA_E_ARG
    bad_ix = swa.IndexStruct(None, 3, 100, FAKE, FAKE, None, 0, 2, 16)      # full layer, no req_to_token
    assert decode(swa, ly, bad_ix, table=None, indptr=None, window=-1) == E.SWA_E_ARG
    # a mapping without the window table: the kernels would read full-pool
    # slots from this pool, so the call is refused
    assert decode(swa, ly, ix, table=None, indptr=None) == E.SWA_E_ARG
    assert decode(swa, ly, ix, table=None, indptr=None, window=-1) == E.SWA_E_ARG
    # the softmax scale must be a positive finite number
    for bad in (0.0, -0.088, float("nan"), float("inf")):
        assert decode(swa, ly, ix, scale=bad) == E.SWA_E_ARG
    assert lib_fused_scale(swa, ly, ix, 0.0) == E.SWA_E_ARG
    assert lib_fused_scale(swa, ly, ix, -1.0) == E.SWA_E_ARG


def lib_fused_scale(swa, ly, ix, scale):
    return swa.lib.swa_decode_store(FAKE, 1, 64, ctypes.byref(ly), ctypes.byref(ix), FAKE, FAKE, 1000, 128, None,
                                    scale, FAKE, FAKE, FAKE, 1, FAKE, 0, None)


def test_empty_batch_launches_nothing(swa):
    """Batch 0 (and an extend with no new tokens) passes the argument checks with
    NULL buffers and returns before any device call, so it runs without a GPU."""
    E, lib = swa, swa.lib
    ly = layer(swa)
    empty = index(swa, batch=0)
    assert decode(swa, ly, empty, q=None, out=None) == E.SWA_OK
    assert decode(swa, ly, empty, q=None, out=None, splits=4) == E.SWA_OK   # no workspace for no requests
    assert decode(swa, ly, empty, window=-2) == E.SWA_E_ARG                  # the checks still apply
    assert decode(swa, layer(swa, head_dim=64), empty) == E.SWA_E_SHAPE
    assert lib.swa_decode_store(None, 1, 64, ctypes.byref(ly), ctypes.byref(empty), FAKE, FAKE, 0, 128, None, 0.088,
                                None, None, None, 1, None, 0, None) == E.SWA_OK
    assert lib.swa_decode_store(None, 1, 64, ctypes.byref(ly), ctypes.byref(empty), FAKE, FAKE, 0, 300, None, 0.088,
                                None, None, None, 1, None, 0, None) == E.SWA_E_SHAPE
    for ix, qo, pre in ((empty, None, None), (index(swa), FAKE, FAKE)):
        assert lib.swa_extend(None, 1, 64, qo, pre, 0, ctypes.byref(ly), ctypes.byref(ix), FAKE, FAKE, 1000, 128,
                              None, 0.088, None, 0, None) == E.SWA_OK
        assert lib.swa_extend_chunked(None, 1, 64, qo, pre, 0, ctypes.byref(ly), ctypes.byref(ix), FAKE, FAKE, 1000,
                                      128, 64, None, 0.088, None, 0, None) == E.SWA_OK


def test_extend_argument_errors(swa):
    E = swa
    ly, ix = layer(swa), index(swa)

    def ext(ly=ly, ix=ix, q_dtype=1, out_dtype=0, total=100, qo=FAKE, pre=FAKE, window=128, table=FAKE, indptr=FAKE,
            scale=0.088):
        return swa.lib.swa_extend(FAKE, q_dtype, 64, qo, pre, total, ctypes.byref(ly), ctypes.byref(ix), table, indptr,
                                  1000, window, None, scale, FAKE, out_dtype, None)

    assert ext(ly=layer(swa, dtype=2)) == E.SWA_E_DTYPE   # extend takes bf16 K/V
    assert ext(q_dtype=0) == E.SWA_E_DTYPE
    assert ext(ly=layer(swa, head_dim=256)) == E.SWA_E_SHAPE
    assert ext(qo=None) == E.SWA_E_ARG
    assert ext(pre=None) == E.SWA_E_ARG
    assert ext(total=-1) == E.SWA_E_ARG
    assert ext(total=1 << 31) == E.SWA_E_SHAPE
    assert ext(window=-3) == E.SWA_E_ARG
    assert ext(table=None, indptr=None) == E.SWA_E_ARG        # a mapping needs the window table
    for bad in (0.0, -1.0, float("nan")):
        assert ext(scale=bad) == E.SWA_E_ARG


def test_store_and_translate_argument_errors(swa):
    E = swa
    lib = swa.lib
    ly = layer(swa)
    # dtype pairs: e4m3 input and bf16 -> f32 are not supported
    assert lib.swa_kv_store(ctypes.byref(layer(swa, dtype=1)), FAKE, 4, FAKE, FAKE, 2, None) == E.SWA_E_DTYPE
    assert lib.swa_kv_store(ctypes.byref(layer(swa, dtype=0)), FAKE, 4, FAKE, FAKE, 1, None) == E.SWA_E_DTYPE
    assert lib.swa_kv_store(ctypes.byref(layer(swa, kv_heads=1, head_dim=4)), FAKE, 4, FAKE, FAKE, 1,
                            None) == E.SWA_E_SHAPE
    assert lib.swa_kv_store(ctypes.byref(ly), FAKE, -1, FAKE, FAKE, 1, None) == E.SWA_E_ARG
    assert lib.swa_kv_store(ctypes.byref(ly), None, 4, FAKE, FAKE, 1, None) == E.SWA_E_ARG
    assert lib.swa_kv_store(ctypes.byref(ly), FAKE, 4, FAKE + 8, FAKE, 1, None) == E.SWA_E_ARG
    assert lib.swa_kv_store(None, FAKE, 4, FAKE, FAKE, 1, None) == E.SWA_E_ARG
    assert lib.swa_kv_store(ctypes.byref(ly), FAKE, 0, FAKE, FAKE, 1, None) == E.SWA_OK  # empty: no launch
    assert lib.swa_translate_loc(FAKE, -1, FAKE, 10, FAKE + 64, None) == E.SWA_E_ARG
    assert lib.swa_translate_loc(FAKE, 5, FAKE, 1, FAKE + 64, None) == E.SWA_E_ARG
    assert lib.swa_translate_loc(FAKE, 5, FAKE, 10, FAKE, None) == E.SWA_E_ARG     # aliasing
    assert lib.swa_translate_loc(None, 0, None, 0, None, None) == E.SWA_OK         # empty: no launch
    ix = index(swa)
    assert lib.swa_translate_window(ctypes.byref(ix), -2, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window(ctypes.byref(ix), 128, None, None, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window(ctypes.byref(ix), 128, None, FAKE, None, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window(None, 128, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG


def test_binding_rejects_host_tensors(swa):
    import torch
    a = torch.zeros(4, dtype=torch.int64)
    with pytest.raises(ValueError):
        swa.swa_translate_loc(a, torch.zeros(10, dtype=torch.int64), torch.zeros(4, dtype=torch.int64))



def test_validate_argument_errors(swa):
    lib, E = swa.lib, swa
    ix = index(swa)
    rep = swa.ValidateReportStruct()
    need = lib.swa_validate_workspace_bytes(1000)
    assert need == 128 + (1000 + 31) // 32 * 4
    assert lib.swa_validate_workspace_bytes(-1) == 0

    def val(ix=ix, window=128, pre=None, rows=1000, loc=FAKE, n=8, ws=FAKE, ws_bytes=need, report=rep, qo=None,
            total_q=0):
        return lib.swa_validate(ctypes.byref(ix), window, pre, qo, total_q, rows, loc, n, ws, ws_bytes,
                                None if report is None else ctypes.byref(report), None)

    assert val(report=None) == E.SWA_E_ARG
    assert val(window=-2) == E.SWA_E_ARG
    assert val(rows=-1) == E.SWA_E_ARG
    assert val(n=-1) == E.SWA_E_ARG
    assert val(loc=None) == E.SWA_E_ARG                       # locs counted but not given
    assert val(ws=None) == E.SWA_E_WORKSPACE
    assert val(ws=FAKE + 8) == E.SWA_E_WORKSPACE              # misaligned
    assert val(ws_bytes=need - 4) == E.SWA_E_WORKSPACE
    assert val(qo=FAKE, total_q=-1) == E.SWA_E_ARG
    no_page = swa.IndexStruct(FAKE, 3, 100, FAKE, FAKE, FAKE, 50, 2, 0)
    assert val(ix=no_page) == E.SWA_E_ARG


def test_decode_store_argument_errors(swa):
    lib, E = swa.lib, swa
    ly, ix = layer(swa), index(swa)

    def fused(window=128, loc=FAKE, new_dtype=1, q_dtype=1, kn=FAKE, ly=ly):
        return lib.swa_decode_store(FAKE, q_dtype, 64, ctypes.byref(ly), ctypes.byref(ix), FAKE, FAKE, 1000, window,
                                    None, 0.088, loc, kn, FAKE, new_dtype, FAKE, 0, None)

    assert fused(loc=None) == E.SWA_E_ARG
    assert fused(kn=None) == E.SWA_E_ARG
    assert fused(kn=FAKE + 8) == E.SWA_E_ARG            # misaligned new rows
    assert fused(new_dtype=0) == E.SWA_E_DTYPE          # f32 new rows: use the two calls
    assert fused(window=-1) == E.SWA_E_SHAPE            # full layers: split-K, no fused store
    assert fused(window=300) == E.SWA_E_SHAPE           # beyond the one-split window kernel
    assert fused(q_dtype=0, ly=layer(swa, dtype=0)) == E.SWA_E_DTYPE


def test_evict_argument_errors(swa):
    lib, E = swa.lib, swa
    ix = index(swa)
    # int32 counts, ranges (2) and one base per chunk of >= 2048 positions starting at page boundaries,
    # rounded up to 8 bytes, then one int64 per candidate: stride // page + 2 per request
    assert lib.swa_evict_workspace_bytes(5, 4096, 16) == 104 + 5 * (4096 // 16 + 2) * 8   # 100 -> 104
    assert lib.swa_evict_workspace_bytes(2, 100, 3) == 32 + 2 * (100 // 3 + 2) * 8       # chunk 2049
    assert lib.swa_evict_workspace_bytes(1, 4097, 4096) == 24 + 1 * (4097 // 4096 + 2) * 8  # chunk 4096; 20 -> 24
    assert lib.swa_evict_workspace_bytes(0, 4096, 16) == 0
    need = lib.swa_evict_workspace_bytes(2, 100, 16)

    def ev(ix=ix, mp=FAKE, pre=FAKE, evd=FAKE, window=128, mode=0, interval=0, pages=FAKE, cap=10, count=FAKE,
           ws=FAKE, ws_bytes=need):
        return lib.swa_evict(ctypes.byref(ix), mp, pre, None, evd, window, mode, interval, pages, cap, count, ws,
                             ws_bytes, None)

    assert ev(mp=None) == E.SWA_E_ARG
    assert ev(count=None) == E.SWA_E_ARG
    assert ev(pre=None) == E.SWA_E_ARG
    assert ev(evd=None) == E.SWA_E_ARG
    assert ev(window=-1) == E.SWA_E_ARG                 # full layers release nothing
    assert ev(mode=2) == E.SWA_E_ARG
    assert ev(interval=-1) == E.SWA_E_ARG
    assert ev(cap=-1) == E.SWA_E_ARG
    assert ev(pages=None) == E.SWA_E_ARG                # a capacity with no buffer
    assert ev(ws=None) == E.SWA_E_WORKSPACE
    assert ev(ws_bytes=need - 4) == E.SWA_E_WORKSPACE
    assert ev(ws=FAKE + 4) == E.SWA_E_WORKSPACE  # int64 values need 8-byte alignment
    assert ev(ws=FAKE + 2) == E.SWA_E_WORKSPACE         # misaligned
    short_map = swa.IndexStruct(FAKE, 3, 100, FAKE, FAKE, None, 1, 2, 16)
    assert ev(ix=short_map) == E.SWA_E_ARG              # a mapping needs its sentinel entry
    long_rows = swa.IndexStruct(FAKE, 3, 65535 * 2048 + 1, FAKE, FAKE, None, 50, 2, 16)
    assert ev(ix=long_rows, ws_bytes=1 << 40) == E.SWA_E_SHAPE


def test_alloc_pages_needed_on_host(swa):
    lib = swa.lib
    pre = np.array([6, 0, 8, 3], np.int32)
    seq = np.array([15, 5, 9, 4], np.int32)
    # ceil(15/4)-ceil(6/4) + ceil(5/4) + ceil(9/4)-ceil(8/4) + ceil(4/4)-ceil(3/4) = 2 + 2 + 1 + 0
    assert lib.swa_alloc_pages_needed(pre.ctypes.data, seq.ctypes.data, 4, 4) == 5
    dec = np.array([1, 4, 5, 9, 2], np.int32)   # decode: a page opens where seq - 1 is a multiple of 4
    assert lib.swa_alloc_pages_needed(None, dec.ctypes.data, 5, 4) == 3
    assert lib.swa_alloc_pages_needed(None, None, 2, 4) == -1
    assert lib.swa_alloc_pages_needed(None, dec.ctypes.data, 5, 0) == -1


def test_alloc_argument_errors_and_no_space(swa):
    lib, E = swa.lib, swa
    full = swa.FreeListStruct(FAKE, 100)
    sl = swa.FreeListStruct(FAKE, 100)

    def ext(batch=2, page=16, pre=FAKE, seq=FAKE, last=FAKE, fl=full, sw=sl, mp=FAKE, map_len=50, n=64,
            pre_h=None, seq_h=None, out=FAKE):
        return lib.swa_alloc_extend(batch, page, pre, seq, last, None if fl is None else ctypes.byref(fl),
                                    None if sw is None else ctypes.byref(sw), mp, map_len, n, pre_h, seq_h, out, FAKE,
                                    None, None)

    assert ext(page=0) == E.SWA_E_ARG
    assert ext(batch=-1) == E.SWA_E_ARG
    assert ext(n=-1) == E.SWA_E_ARG
    assert ext(fl=None) == E.SWA_E_ARG
    assert ext(pre=None) == E.SWA_E_ARG
    assert ext(last=None) == E.SWA_E_ARG
    assert ext(out=None) == E.SWA_E_ARG
    assert ext(mp=None) == E.SWA_E_ARG                       # two pools need the mapping
    assert ext(map_len=1) == E.SWA_E_ARG
    assert ext(fl=swa.FreeListStruct(None, 5)) == E.SWA_E_ARG
    # the bound 64/16 + 2 + 1 = 7 pages is not provable against a 6-page list and no host lengths are given
    assert ext(sw=swa.FreeListStruct(FAKE, 6)) == E.SWA_E_NOSPACE
    # the exact count (host copies) needs 9 pages: still too many
    pre_h = np.array([0, 20], np.int32)
    seq_h = np.array([64, 84], np.int32)
    assert ext(sw=swa.FreeListStruct(FAKE, 6), pre_h=pre_h.ctypes.data, seq_h=seq_h.ctypes.data) == E.SWA_E_NOSPACE

    def dec(batch=2, fl=full, sw=sl, seq_h=None, out=FAKE, mp=FAKE):
        return lib.swa_alloc_decode(batch, 16, FAKE, FAKE, ctypes.byref(fl), None if sw is None else ctypes.byref(sw),
                                    mp, 50, seq_h, out, None, None, None)

    assert dec(out=None) == E.SWA_E_ARG
    assert dec(mp=None) == E.SWA_E_ARG
    assert dec(fl=swa.FreeListStruct(FAKE, -1)) == E.SWA_E_ARG
    assert dec(sw=swa.FreeListStruct(FAKE, 1)) == E.SWA_E_NOSPACE           # bound: 2 pages
    two = np.array([17, 33], np.int32)                                      # both open a page
    assert dec(sw=swa.FreeListStruct(FAKE, 1), seq_h=two.ctypes.data) == E.SWA_E_NOSPACE


def test_unified_views_on_host_match_the_oracle_builder(swa):
    """swa_unified_layer_views is host arithmetic only: its view pointers must
    start where the oracle's strided builder starts each layer's block."""
    from oracle import swa_oracle as O
    lib, E = swa.lib, swa
    L, H, D, P, pages, anchor = 5, 8, 128, 16, 37, 4096
    g = O.unified_geometry(L, H, D, 2, P, pages)
    need = lib.swa_unified_pool_bytes(L, H, D, swa.SWA_BF16, P, pages)
    assert need == g["total_bytes"] + g["tail_pad"]
    views = (swa.KvLayerStruct * L)()
    raw = 1 << 20   # never dereferenced
    assert lib.swa_unified_layer_views(raw, anchor + need, anchor, L, H, D, swa.SWA_BF16, P, pages, 1.0, 1.0,
                                       views) == E.SWA_OK
    for layer in range(L):
        assert views[layer].k == raw + O.unified_view_base(anchor, layer, 0, g["row_bytes"], P)
        assert views[layer].v == raw + O.unified_view_base(anchor, layer, 1, g["row_bytes"], P)
        assert views[layer].rows == g["n_rows"] and views[layer].kv_heads == H and views[layer].dtype == swa.SWA_BF16
    # one byte short of the tail pad: the last views would run past the buffer
    assert lib.swa_unified_layer_views(raw, anchor + need - 1, anchor, L, H, D, swa.SWA_BF16, P, pages, 1.0, 1.0,
                                       views) == E.SWA_E_SHAPE
    assert lib.swa_unified_layer_views(raw, 1 << 40, 8, L, H, D, swa.SWA_BF16, P, pages, 1.0, 1.0,
                                       views) == E.SWA_E_ARG       # anchor not 16-aligned
    assert lib.swa_unified_layer_views(raw, 1 << 40, 0, L, H, D, 7, P, pages, 1.0, 1.0, views) == E.SWA_E_DTYPE
    # kernel-facing rows reach 2^31: refused (int32 index buffers)
    big = (1 << 31) // (2 * L * P) + 1
    assert lib.swa_unified_layer_views(raw, 1 << 62, 0, L, H, D, swa.SWA_BF16, P, big, 1.0, 1.0,
                                       views) == E.SWA_E_SHAPE
    assert lib.swa_unified_pool_bytes(0, H, D, swa.SWA_BF16, P, pages) == -1


def test_unified_translate_argument_errors(swa):
    lib, E = swa.lib, swa
    assert lib.swa_translate_kernel_ids(FAKE, 10, FAKE, 4, 0, 2, FAKE, None) == E.SWA_E_ARG
    assert lib.swa_translate_kernel_ids(FAKE, 10, FAKE, 4, 16, 0, FAKE, None) == E.SWA_E_ARG
    assert lib.swa_translate_kernel_ids(FAKE, 10, None, 4, 16, 2, FAKE, None) == E.SWA_E_ARG
    assert lib.swa_translate_kernel_ids(None, 10, FAKE, 4, 16, 2, FAKE, None) == E.SWA_E_ARG
    ix = index(swa, map_ptr=None)

    def win(v2p=FAKE, n_pages=100, mult=64, window=128, table=FAKE, cap=1000):
        return lib.swa_translate_window_unified(ctypes.byref(ix), v2p, n_pages, mult, window, None, table, FAKE, cap,
                                                None)

    assert win(v2p=None) == E.SWA_E_ARG
    assert win(mult=0) == E.SWA_E_ARG
    assert win(window=-2) == E.SWA_E_ARG
    assert win(table=None) == E.SWA_E_ARG
    assert win(n_pages=(1 << 31) // (16 * 64) + 1) == E.SWA_E_SHAPE     # ids would pass 2^31


def test_variant_argument_errors(swa):
    lib, E = swa.lib, swa
    ix = index(swa)
    assert lib.swa_translate_window_chunked(ctypes.byref(ix), 128, -1, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window_chunked(ctypes.byref(ix), -2, 64, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window_chunked(ctypes.byref(ix), -1, 64, None, FAKE, None, 10, None) == E.SWA_E_ARG
    ring_ix = swa.IndexStruct(None, 8, 100, FAKE, FAKE, None, 0, 2, 16)
    assert lib.swa_translate_window_ring(ctypes.byref(ring_ix), 0, 128, 0, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window_ring(ctypes.byref(ring_ix), 144, -2, 0, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_translate_window_ring(ctypes.byref(ring_ix), (1 << 31) // 8 + 1, 128, 0, None, FAKE, FAKE, 10,
                                         None) == E.SWA_E_SHAPE
    no_rows = swa.IndexStruct(None, 8, 100, None, FAKE, None, 0, 2, 16)
    assert lib.swa_translate_window_ring(ctypes.byref(no_rows), 144, 128, 0, None, FAKE, FAKE, 10, None) == E.SWA_E_ARG
    assert lib.swa_ring_locs(ctypes.byref(ring_ix), 0, None, FAKE, 2, None) == E.SWA_E_ARG
    assert lib.swa_ring_locs(ctypes.byref(ring_ix), 144, None, None, 2, None) == E.SWA_E_ARG
    ly = layer(swa)
    assert lib.swa_extend_chunked(FAKE, 1, 64, FAKE, FAKE, 16, ctypes.byref(ly), ctypes.byref(ix), None, None, 0, 128,
                                  -1, None, 0.088, FAKE, 0, None) == E.SWA_E_ARG
    one_pool = index(swa, map_ptr=None)
    assert lib.swa_extend_chunked(FAKE, 0, 64, FAKE, FAKE, 16, ctypes.byref(ly), ctypes.byref(one_pool), None, None, 0,
                                  128, 64, None, 0.088, FAKE, 0, None) == E.SWA_E_DTYPE
    assert lib.swa_extend_chunked(FAKE, 1, 64, FAKE, FAKE, 16, ctypes.byref(ly), ctypes.byref(ix), None, None, 0, 128,
                                  64, None, 0.088, FAKE, 0, None) == E.SWA_E_ARG   # a mapping needs the table


def test_decode_workspace_bytes_bounds_every_plan(swa):
    lib = swa.lib
    for B, Hq, Hkv, keys in ((32, 64, 4, 32768), (1, 8, 8, 512), (3, 16, 2, 5000), (256, 64, 8, 65536)):
        bound = lib.swa_decode_workspace_bytes(B, Hq, 128, keys)
        for T in (t for t in (1, 100, 511, 512, 513, keys // 2, keys) if t <= keys):
            ns, ws = ctypes.c_int32(), ctypes.c_size_t()
            assert lib.swa_decode_plan(B, Hq, Hkv, 128, -1, T, ctypes.byref(ns), ctypes.byref(ws)) == swa.SWA_OK
            assert ws.value <= bound
    assert lib.swa_decode_workspace_bytes(4, 8, 128, 512) == 0          # one split: no workspace
    assert lib.swa_decode_workspace_bytes(4, 8, 64, 5000) == 0          # head_dim other than 128


def step_struct(swa, n_swa=3, n_full=2, mapping=None, window=128, q=True, store=False, swa_loc=True,
                full_kv=4):
    """A decode-step descriptor over fake device pointers (never dereferenced:
    every case below fails its checks, or has an empty batch, before a launch)."""
    mapping = [(0, 0), (0, 1), (1, 1), (1, 0), (2, 1)] if mapping is None else mapping
    n = len(mapping)
    keep = []

    def arr(t, vals):
        a = (t * max(len(vals), 1))(*vals)
        keep.append(a)
        return ctypes.cast(a, ctypes.POINTER(t))

    m = arr(swa.LayerMapStruct, [swa.LayerMapStruct(p, s) for p, s in mapping])
    full = arr(swa.KvLayerStruct, [layer(swa, kv_heads=full_kv) for _ in range(n_full)])
    swal = arr(swa.KvLayerStruct, [layer(swa) for _ in range(n_swa)])
    ptrs = arr(ctypes.c_void_p, [FAKE] * n)
    st = swa.DecodeStepStruct(n, m, full, n_full, swal, n_swa, window, 64, 1, 0, ptrs if q else None, ptrs, None,
                              0.088, FAKE if store else None, FAKE if (store and swa_loc) else None,
                              ptrs if store else None, ptrs if store else None)
    st._keep = keep
    return st


def test_decode_step_argument_errors(swa):
    lib, E = swa.lib, swa
    ix = index(swa)

    def step(st, ws=None, ws_bytes=0, table=FAKE, indptr=FAKE, ix=ix, max_seq=32768):
        return lib.swa_decode_step(ctypes.byref(st), ctypes.byref(ix), max_seq, table, indptr, 1000, ws, ws_bytes,
                                   None)

    need = lib.swa_decode_step_workspace_bytes(ctypes.byref(step_struct(swa)), ctypes.byref(ix), 32768)
    ns, ws = ctypes.c_int32(), ctypes.c_size_t()
    assert lib.swa_decode_plan(2, 64, 4, 128, -1, 32768, ctypes.byref(ns), ctypes.byref(ws)) == E.SWA_OK
    assert need == ws.value > 0                                     # the full layers' split-K plan
    assert lib.swa_decode_step_workspace_bytes(ctypes.byref(step_struct(swa, mapping=[(0, 1)])), ctypes.byref(ix),
                                               32768) == 0           # SWA layers only: no workspace
    assert step(step_struct(swa, mapping=[(3, 1)])) == E.SWA_E_ARG   # SWA pool has 3 layers
    assert step(step_struct(swa, mapping=[(2, 0)])) == E.SWA_E_ARG   # full pool has 2 layers
    assert step(step_struct(swa, mapping=[(0, 2)])) == E.SWA_E_ARG   # is_swa is 0 or 1
    assert step(step_struct(swa, mapping=[(-1, 1)])) == E.SWA_E_ARG
    assert step(step_struct(swa, window=-1)) == E.SWA_E_ARG
    assert step(step_struct(swa, q=False)) == E.SWA_E_ARG
    assert step(step_struct(swa, store=True, swa_loc=False), ws=FAKE, ws_bytes=need) == E.SWA_E_ARG
    assert step(step_struct(swa)) == E.SWA_E_WORKSPACE               # full layers need the split workspace
    assert step(step_struct(swa), ws=FAKE, ws_bytes=need - 16) == E.SWA_E_WORKSPACE
    assert step(step_struct(swa), ws=FAKE, ws_bytes=need, table=None) == E.SWA_E_ARG
    assert step(step_struct(swa, full_kv=3), ws=FAKE, ws_bytes=need) == E.SWA_E_SHAPE   # 64 q over 3 kv heads
    # an empty batch passes the checks and launches nothing
    assert step(step_struct(swa), ix=index(swa, batch=0), ws=None) == E.SWA_OK
    assert step(step_struct(swa, mapping=[])) == E.SWA_OK


def test_decode_noalloc_host_checks(swa):
    """The no-allocation decode checks its arguments like swa_decode, and a plan
    whose split partials exceed the static scratch is refused before any
    device call (so these run without a GPU)."""
    lib, E = swa.lib, swa
    ly = layer(swa, kv_heads=4)
    full = index(swa, map_ptr=None)

    def nd(ix=full, splits=8, q=FAKE, window=-1, scale=0.088, q_heads=64):
        return lib.swa_decode_noalloc(q, 1, q_heads, ctypes.byref(ly), ctypes.byref(ix), None, None, 0, window, None,
                                      scale, FAKE, 0, splits, None)

    assert nd(q=None) == E.SWA_E_ARG
    assert nd(window=-2) == E.SWA_E_ARG
    assert nd(scale=0.0) == E.SWA_E_ARG
    assert nd(q_heads=24) == E.SWA_E_SHAPE
    assert nd(splits=0) == E.SWA_E_ARG
    # 32 MiB holds batch * q_heads * splits <= 64527 partials of 520 bytes
    big = swa.IndexStruct(FAKE, 3, 100, FAKE, FAKE, None, 0, 1024, 16)
    assert nd(ix=big, splits=8) == E.SWA_E_WORKSPACE       # 1024 x 64 x 8 partials
    assert nd(ix=index(swa, batch=0, map_ptr=None)) == E.SWA_OK   # empty batch: nothing launched


def test_probe_argument_errors(swa):
    lib, E = swa.lib, swa
    assert lib.swa_probe_read(None, 1024, FAKE, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_read(FAKE, 1024, None, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_read(FAKE, 0, FAKE, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_read(FAKE, 1000, FAKE, 8, None) == E.SWA_E_ARG       # not a multiple of 16
    assert lib.swa_probe_read(FAKE + 8, 1024, FAKE, 8, None) == E.SWA_E_ARG   # not 16-aligned
    assert lib.swa_probe_read(FAKE, 1024, FAKE, 0, None) == E.SWA_E_ARG
    assert lib.swa_probe_read(FAKE, 1024, FAKE, 65536, None) == E.SWA_E_ARG
    assert lib.swa_probe_copy(None, FAKE, 1024, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_copy(FAKE, None, 1024, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_copy(FAKE, FAKE + 512, 1024, 8, None) == E.SWA_E_ARG   # overlapping
    assert lib.swa_probe_copy(FAKE + 1024, FAKE, 1024 + 16, 8, None) == E.SWA_E_ARG  # overlapping the other way
    assert lib.swa_probe_copy(FAKE, FAKE + 4096, 1000, 8, None) == E.SWA_E_ARG  # not a multiple of 16
    assert lib.swa_probe_copy(FAKE + 8, FAKE + 4096, 1024, 8, None) == E.SWA_E_ARG
    assert lib.swa_probe_copy(FAKE, FAKE + 4096, 1024, 0, None) == E.SWA_E_ARG
    assert lib.swa_probe_mfma(None, 8, 1, None) == E.SWA_E_ARG
    assert lib.swa_probe_mfma(FAKE, 0, 1, None) == E.SWA_E_ARG
    assert lib.swa_probe_mfma(FAKE, 8, 0, None) == E.SWA_E_ARG
