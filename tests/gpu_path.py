"""Helpers for the GPU parity tests: upload a seeded workload, run the HIP path
through the C-ABI binding, and compute the CPU oracle on the same inputs.

Only torch is used to move data (allocation, fills, copies, index scatter of
the generator's values); every step of the path runs in libswa."""

from __future__ import annotations

import math
import sys

import numpy as np
import torch

from oracle import codecs
from oracle import swa_oracle as O
from sliding_window_attention_swa_amd import workloads as WL

TOL = {"f32": 1e-5, "bf16": 2e-2, "e4m3": 6e-2}
TORCH_STORE = {"f32": torch.float32, "bf16": torch.bfloat16, "e4m3": torch.uint8}


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def bits_to_device(bits: np.ndarray, dtype: str, device="cuda") -> torch.Tensor:
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.float32)).to(device)
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).to(device).view(torch.bfloat16)
    if dtype == "e4m3":
        return torch.from_numpy(np.ascontiguousarray(bits, dtype=np.uint8)).to(device)
    raise ValueError(dtype)


def device_to_bits(t: torch.Tensor) -> np.ndarray:
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def pool_to_device(pool: WL.SparsePool, device="cuda") -> torch.Tensor:
    rows, H, D = pool.shape
    t = torch.empty((rows, H, D), dtype=TORCH_STORE[pool.dtype], device=device)
    nan = WL.NAN_BITS[pool.dtype]
    if pool.dtype == "bf16":
        t.view(torch.int16).fill_(int(np.int16(nan.view(np.int16))))
    elif pool.dtype == "e4m3":
        t.fill_(int(nan))
    else:
        t.fill_(float("nan"))
    used = pool.written_rows()
    if used.size:
        vals = pool[used]
        t[torch.from_numpy(used).to(device)] = bits_to_device(vals, pool.dtype, device)
    return t


class DeviceWorkload:
    """Device copies of a Workload's tensors (index tables, pools, Q, sinks)."""

    def __init__(self, wl: WL.Workload, device="cuda"):
        from sliding_window_attention_swa_amd import swa
        self.wl = wl
        self.r2t = torch.from_numpy(wl.req_to_token).to(device)
        self.rows = torch.from_numpy(wl.req_pool_idx).to(device)
        self.lens = torch.from_numpy(wl.seq_lens.astype(np.int32)).to(device)
        self.map = None if wl.full_to_swa is None else torch.from_numpy(wl.full_to_swa).to(device)
        self.k = pool_to_device(wl.pool_k, device)
        self.v = pool_to_device(wl.pool_v, device)
        self.q = bits_to_device(wl.q, wl.q_dtype, device)
        self.sinks = None if wl.sinks is None else torch.from_numpy(wl.sinks).to(device)
        self.index = swa.IndexTables(self.r2t, self.rows, self.lens, self.map, wl.page_size)
        self.layer = swa.KvLayer(self.k, self.v)
        self.prefix = None if wl.prefix_lens is None else torch.from_numpy(wl.prefix_lens).to(device)
        self.qo = None if wl.qo_indptr is None else torch.from_numpy(wl.qo_indptr).to(device)


def run_store(dw: DeviceWorkload, in_dtype="bf16"):
    """translate_loc of the new tokens' full locs, then kv_store at the SWA
    slots (or at the full locs on a single-pool layer)."""
    from sliding_window_attention_swa_amd import swa
    wl = dw.wl
    full = torch.from_numpy(wl.new_full_loc).cuda()
    if dw.map is not None:
        loc = torch.empty_like(full)
        swa.swa_translate_loc(full, dw.map, loc)
    else:
        loc = full
    kn = bits_to_device(wl.new_k, wl.new_dtype)
    vn = bits_to_device(wl.new_v, wl.new_dtype)
    swa.swa_kv_store(dw.layer, loc, kn, vn)
    return loc


def run_decode_store(dw: DeviceWorkload, out_dtype="f32"):
    """The fused call: the new tokens' store and the decode in one launch."""
    from sliding_window_attention_swa_amd import swa
    wl = dw.wl
    B = wl.batch
    full = torch.from_numpy(wl.new_full_loc).cuda()
    loc = torch.empty_like(full)
    swa.swa_translate_loc(full, dw.map, loc)
    table = torch.empty(max(B * (wl.window + 1), 1), dtype=torch.int32, device="cuda")
    indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
    swa.swa_translate_window(dw.index, wl.window, table, indptr)
    out = torch.empty((B, wl.q_heads, wl.head_dim), dtype=TORCH_STORE[out_dtype], device="cuda")
    swa.swa_decode_store(dw.q, dw.layer, dw.index, wl.window, out, loc, bits_to_device(wl.new_k, wl.new_dtype),
                         bits_to_device(wl.new_v, wl.new_dtype), sinks=dw.sinks, slot_table=table,
                         table_indptr=indptr)
    torch.cuda.synchronize()
    return out


def run_decode(dw: DeviceWorkload, out_dtype="f32", num_splits=None, use_table=True, max_seq=None):
    from sliding_window_attention_swa_amd import swa
    wl = dw.wl
    B = wl.batch
    table = indptr = None
    if use_table and wl.window >= 0 and dw.map is not None:
        cap = B * (wl.window + 1)
        table = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
        indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        swa.swa_translate_window(dw.index, wl.window, table, indptr)
    if num_splits is None:
        num_splits, ws_bytes = swa.swa_decode_plan(B, wl.q_heads, wl.kv_heads, wl.head_dim, wl.window,
                                                   max_seq or int(wl.seq_lens.max()))
    ws = None
    if num_splits > 1:
        ws = torch.empty(B * wl.q_heads * num_splits * (2 + wl.head_dim), dtype=torch.float32, device="cuda")
    out = torch.empty((B, wl.q_heads, wl.head_dim), dtype=TORCH_STORE[out_dtype], device="cuda")
    swa.swa_decode(dw.q, dw.layer, dw.index, wl.window, out, sinks=dw.sinks, slot_table=table, table_indptr=indptr,
                   num_splits=num_splits, workspace=ws, use_map=dw.map is not None)
    torch.cuda.synchronize()
    return out


def run_extend(dw: DeviceWorkload, out_dtype="f32", use_table=True, chunk=0):
    """swa_extend (chunk > 0: swa_extend_chunked over a chunked table)."""
    from sliding_window_attention_swa_amd import swa
    wl = dw.wl
    B = wl.batch
    table = indptr = None
    use_map = dw.map is not None
    if use_table:
        cap = int(wl.seq_lens.astype(np.int64).sum())   # at least every window
        table = torch.empty(max(cap, 1), dtype=torch.int32, device="cuda")
        indptr = torch.empty(B + 1, dtype=torch.int32, device="cuda")
        if chunk:
            swa.swa_translate_window_chunked(dw.index, wl.window, chunk, table, indptr, prefix_lens=dw.prefix,
                                             use_map=use_map)
        else:
            swa.swa_translate_window(dw.index, wl.window, table, indptr, prefix_lens=dw.prefix, use_map=use_map)
    out = torch.empty((wl.q.shape[0], wl.q_heads, wl.head_dim), dtype=TORCH_STORE[out_dtype], device="cuda")
    if chunk:
        swa.swa_extend_chunked(dw.q, dw.qo, dw.prefix, dw.layer, dw.index, wl.window, chunk, out, sinks=dw.sinks,
                               slot_table=table, table_indptr=indptr, use_map=use_map)
    else:
        swa.swa_extend(dw.q, dw.qo, dw.prefix, dw.layer, dw.index, wl.window, out, sinks=dw.sinks,
                       slot_table=table, table_indptr=indptr, use_map=use_map)
    torch.cuda.synchronize()
    return out


def oracle_pools_after_store(wl: WL.Workload):
    """The oracle's own store of the new tokens (its translation and codecs)."""
    if wl.new_full_loc is None:
        return wl.pool_k, wl.pool_v
    loc = O.translate_loc(wl.new_full_loc, wl.full_to_swa) if wl.full_to_swa is not None else wl.new_full_loc
    return O.kv_store(wl.pool_k, wl.pool_v, loc, wl.new_k, wl.new_v, wl.new_dtype, wl.kv_dtype)


def oracle_decode(wl: WL.Workload, only=None, chunk=0):
    pk, pv = oracle_pools_after_store(wl)
    return O.decode(wl.q, wl.q_dtype, pk, pv, wl.kv_dtype, wl.req_to_token, wl.req_pool_idx, wl.seq_lens,
                    wl.full_to_swa, wl.window, wl.sinks, only=only, chunk=chunk)


def oracle_extend(wl: WL.Workload, only=None, chunk=0):
    pk, pv = oracle_pools_after_store(wl)
    return O.extend(wl.q, wl.q_dtype, wl.qo_indptr, wl.prefix_lens, pk, pv, wl.kv_dtype, wl.req_to_token,
                    wl.req_pool_idx, wl.seq_lens, wl.full_to_swa, wl.window, wl.sinks, only=only, chunk=chunk)


def rel_err(got: np.ndarray, ref: np.ndarray) -> float:
    """max |got - ref| / RMS(ref) over the entries the oracle computed."""
    m = ~np.isnan(ref)
    ref_m = ref[m]
    rms = math.sqrt(float(np.mean(ref_m ** 2)))
    return float(np.max(np.abs(got[m].astype(np.float64) - ref_m))) / rms


def check(got_t: torch.Tensor, ref: np.ndarray, tol: float, what: str):
    got = got_t.detach().float().cpu().numpy() if got_t.dtype != torch.float32 else got_t.detach().cpu().numpy()
    m = ~np.isnan(ref)
    assert np.isfinite(got[m]).all(), f"{what}: non-finite output"
    e = rel_err(got, ref)
    say(f"  {what}: max|err|/rms = {e:.3e} (tol {tol:g})")
    assert e <= tol, f"{what}: {e:.3e} > {tol}"
    return e
