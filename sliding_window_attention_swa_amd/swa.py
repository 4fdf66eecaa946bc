"""Thin Python binding of libswa (ctypes).  Argument marshalling only: every
step of the path runs in the library's HIP kernels.  PyTorch supplies device
memory and streams.

The function names are the C names (include/swa.h).  Tensors must be
contiguous CUDA (HIP) tensors of the documented dtypes; the binding checks
device, dtype and contiguity, converts them to pointers and raises SwaError on
a non-zero status.  There is no fallback: if libswa.so is missing the import
of this module fails.
"""

from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import numpy as np
import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libswa.so")

SWA_OK, SWA_E_ARG, SWA_E_DTYPE, SWA_E_SHAPE, SWA_E_NOSPACE, SWA_E_WORKSPACE, SWA_E_HIP = 0, -1, -2, -3, -4, -5, -6
SWA_F32, SWA_BF16, SWA_FP8_E4M3 = 0, 1, 2

# every symbol include/swa.h and include/swa_probe.h declare
EXPORTS = ("swa_pool_config", "swa_translate_loc", "swa_translate_window", "swa_kv_store", "swa_decode_plan",
           "swa_decode", "swa_decode_store", "swa_extend", "swa_validate_workspace_bytes", "swa_validate",
           "swa_evict_workspace_bytes", "swa_evict", "swa_alloc_pages_needed", "swa_alloc_extend",
           "swa_alloc_decode", "swa_unified_pool_bytes", "swa_unified_layer_views", "swa_translate_kernel_ids",
           "swa_translate_window_unified", "swa_translate_window_chunked", "swa_extend_chunked",
           "swa_translate_window_ring", "swa_ring_locs", "swa_decode_workspace_bytes", "swa_decode_step",
           "swa_decode_step_workspace_bytes", "swa_decode_noalloc", "swa_status_string",
           # include/swa_probe.h: measurement probes for the benchmark
           "swa_probe_read", "swa_probe_copy", "swa_probe_mfma")


class SwaError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {status_string(status)} ({status})")
        self.status = status


def _load() -> ctypes.CDLL:
    if not os.path.exists(_LIB_PATH):
        raise ImportError(f"{_LIB_PATH} is missing: build it with `python -m sliding_window_attention_swa_amd.build`")
    return ctypes.CDLL(_LIB_PATH)


lib = _load()


class KvLayerStruct(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("v", ctypes.c_void_p), ("rows", ctypes.c_int64),
                ("kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32), ("dtype", ctypes.c_int32),
                ("k_scale", ctypes.c_float), ("v_scale", ctypes.c_float)]


class IndexStruct(ctypes.Structure):
    _fields_ = [("req_to_token", ctypes.c_void_p), ("r2t_rows", ctypes.c_int64), ("r2t_stride", ctypes.c_int64),
                ("req_pool_idx", ctypes.c_void_p), ("seq_lens", ctypes.c_void_p), ("full_to_swa", ctypes.c_void_p),
                ("map_len", ctypes.c_int64), ("batch", ctypes.c_int32), ("page_size", ctypes.c_int32)]


class LayerMapStruct(ctypes.Structure):
    _fields_ = [("pool_layer", ctypes.c_int32), ("is_swa", ctypes.c_int32)]


class DecodeStepStruct(ctypes.Structure):
    _fields_ = [("n_layers", ctypes.c_int32), ("layers_mapping", ctypes.POINTER(LayerMapStruct)),
                ("full_layers", ctypes.POINTER(KvLayerStruct)), ("n_full_layers", ctypes.c_int32),
                ("swa_layers", ctypes.POINTER(KvLayerStruct)), ("n_swa_layers", ctypes.c_int32),
                ("window", ctypes.c_int32), ("q_heads", ctypes.c_int32), ("q_dtype", ctypes.c_int32),
                ("out_dtype", ctypes.c_int32), ("q", ctypes.POINTER(ctypes.c_void_p)),
                ("out", ctypes.POINTER(ctypes.c_void_p)), ("sinks", ctypes.POINTER(ctypes.c_void_p)),
                ("sm_scale", ctypes.c_float), ("full_loc", ctypes.c_void_p), ("swa_loc", ctypes.c_void_p),
                ("k_new", ctypes.POINTER(ctypes.c_void_p)), ("v_new", ctypes.POINTER(ctypes.c_void_p))]


class FreeListStruct(ctypes.Structure):
    _fields_ = [("pages", ctypes.c_void_p), ("count", ctypes.c_int64)]


VALIDATE_FIELDS = ("bad_requests", "positions", "full_out_of_range", "tombstones", "sentinels", "slot_out_of_range",
                   "store_locs", "store_out_of_range", "store_duplicates", "qo_bad")


class ValidateReportStruct(ctypes.Structure):
    _fields_ = [(f, ctypes.c_int64) for f in VALIDATE_FIELDS]


_i32, _i64, _f32, _f64, _p, _sz = (ctypes.c_int32, ctypes.c_int64, ctypes.c_float, ctypes.c_double, ctypes.c_void_p,
                                   ctypes.c_size_t)
_sig = {
    "swa_pool_config": (_i32, [_i64, _f64, _i32, _i32, _i32, _i64, _i32, _i64, ctypes.POINTER(_i64),
                               ctypes.POINTER(_i64)]),
    "swa_translate_loc": (_i32, [_p, _i64, _p, _i64, _p, _p]),
    "swa_translate_window": (_i32, [ctypes.POINTER(IndexStruct), _i32, _p, _p, _p, _i64, _p]),
    "swa_kv_store": (_i32, [ctypes.POINTER(KvLayerStruct), _p, _i64, _p, _p, _i32, _p]),
    "swa_decode_plan": (_i32, [_i32, _i32, _i32, _i32, _i32, _i64, ctypes.POINTER(_i32), ctypes.POINTER(_sz)]),
    "swa_decode": (_i32, [_p, _i32, _i32, ctypes.POINTER(KvLayerStruct), ctypes.POINTER(IndexStruct), _p, _p, _i64,
                          _i32, _p, _f32, _p, _i32, _i32, _p, _sz, _p]),
    "swa_decode_noalloc": (_i32, [_p, _i32, _i32, ctypes.POINTER(KvLayerStruct), ctypes.POINTER(IndexStruct), _p,
                                  _p, _i64, _i32, _p, _f32, _p, _i32, _i32, _p]),
    "swa_decode_store": (_i32, [_p, _i32, _i32, ctypes.POINTER(KvLayerStruct), ctypes.POINTER(IndexStruct), _p, _p,
                                _i64, _i32, _p, _f32, _p, _p, _p, _i32, _p, _i32, _p]),
    "swa_extend": (_i32, [_p, _i32, _i32, _p, _p, _i64, ctypes.POINTER(KvLayerStruct), ctypes.POINTER(IndexStruct),
                          _p, _p, _i64, _i32, _p, _f32, _p, _i32, _p]),
    "swa_validate_workspace_bytes": (_sz, [_i64]),
    "swa_validate": (_i32, [ctypes.POINTER(IndexStruct), _i32, _p, _p, _i64, _i64, _p, _i64, _p, _sz,
                            ctypes.POINTER(ValidateReportStruct), _p]),
    "swa_evict_workspace_bytes": (_sz, [_i32, _i64, _i32]),
    "swa_evict": (_i32, [ctypes.POINTER(IndexStruct), _p, _p, _p, _p, _i32, _i32, _i32, _p, _i64, _p, _p, _sz, _p]),
    "swa_alloc_pages_needed": (_i64, [_p, _p, _i32, _i32]),
    "swa_alloc_extend": (_i32, [_i32, _i32, _p, _p, _p, ctypes.POINTER(FreeListStruct), ctypes.POINTER(FreeListStruct),
                                _p, _i64, _i64, _p, _p, _p, _p, _p, _p]),
    "swa_alloc_decode": (_i32, [_i32, _i32, _p, _p, ctypes.POINTER(FreeListStruct), ctypes.POINTER(FreeListStruct),
                                _p, _i64, _p, _p, _p, _p, _p]),
    "swa_unified_pool_bytes": (_i64, [_i32, _i32, _i32, _i32, _i32, _i64]),
    "swa_unified_layer_views": (_i32, [_p, _i64, _i64, _i32, _i32, _i32, _i32, _i32, _i64, _f32, _f32,
                                       ctypes.POINTER(KvLayerStruct)]),
    "swa_translate_kernel_ids": (_i32, [_p, _i64, _p, _i64, _i32, _i32, _p, _p]),
    "swa_translate_window_unified": (_i32, [ctypes.POINTER(IndexStruct), _p, _i64, _i32, _i32, _p, _p, _p, _i64,
                                            _p]),
    "swa_translate_window_chunked": (_i32, [ctypes.POINTER(IndexStruct), _i32, _i32, _p, _p, _p, _i64, _p]),
    "swa_extend_chunked": (_i32, [_p, _i32, _i32, _p, _p, _i64, ctypes.POINTER(KvLayerStruct),
                                  ctypes.POINTER(IndexStruct), _p, _p, _i64, _i32, _i32, _p, _f32, _p, _i32, _p]),
    "swa_translate_window_ring": (_i32, [ctypes.POINTER(IndexStruct), _i64, _i32, _i32, _p, _p, _p, _i64, _p]),
    "swa_ring_locs": (_i32, [ctypes.POINTER(IndexStruct), _i64, _p, _p, _i64, _p]),
    "swa_decode_workspace_bytes": (_sz, [_i32, _i32, _i32, _i32]),
    "swa_decode_step_workspace_bytes": (_sz, [ctypes.POINTER(DecodeStepStruct), ctypes.POINTER(IndexStruct), _i64]),
    "swa_decode_step": (_i32, [ctypes.POINTER(DecodeStepStruct), ctypes.POINTER(IndexStruct), _i64, _p, _p, _i64, _p,
                               _sz, _p]),
    "swa_status_string": (ctypes.c_char_p, [_i32]),
    "swa_probe_read": (_i32, [_p, _sz, _p, _i32, _p]),
    "swa_probe_copy": (_i32, [_p, _p, _sz, _i32, _p]),
    "swa_probe_mfma": (_i32, [_p, _i32, _i32, _p]),
}
for _name, (_res, _args) in _sig.items():
    _fn = getattr(lib, _name)
    _fn.restype = _res
    _fn.argtypes = _args


def status_string(status: int) -> str:
    return lib.swa_status_string(status).decode()


def _check(status: int, what: str) -> None:
    if status != SWA_OK:
        raise SwaError(status, what)


_TORCH_DTYPE = {SWA_F32: torch.float32, SWA_BF16: torch.bfloat16, SWA_FP8_E4M3: torch.uint8}


def dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.float32:
        return SWA_F32
    if t.dtype == torch.bfloat16:
        return SWA_BF16
    if t.dtype in (torch.uint8, torch.float8_e4m3fn):
        return SWA_FP8_E4M3
    raise TypeError(f"unsupported tensor dtype {t.dtype}")


def _ptr(t: Optional[torch.Tensor], dtype=None, name="tensor") -> Optional[int]:
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype not in (dtype if isinstance(dtype, tuple) else (dtype,)):
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    return t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream)


@dataclass
class KvLayer:
    """One layer's K and V views of a pool: (rows, kv_heads, head_dim) tensors."""
    k: torch.Tensor
    v: torch.Tensor
    k_scale: float = 1.0
    v_scale: float = 1.0

    def struct(self) -> KvLayerStruct:
        if self.k.shape != self.v.shape or self.k.dim() != 3 or self.k.dtype != self.v.dtype:
            raise ValueError("k and v must be (rows, kv_heads, head_dim) tensors of one dtype")
        return KvLayerStruct(_ptr(self.k, name="k"), _ptr(self.v, name="v"), self.k.shape[0], self.k.shape[1],
                             self.k.shape[2], dtype_code(self.k), self.k_scale, self.v_scale)


@dataclass
class IndexTables:
    """The batch's req_to_token / req_pool_idx / seq_lens / full_to_swa tensors."""
    req_to_token: torch.Tensor
    req_pool_idx: torch.Tensor
    seq_lens: torch.Tensor
    full_to_swa: Optional[torch.Tensor] = None
    page_size: int = 1

    def struct(self, with_map: bool = True) -> IndexStruct:
        m = self.full_to_swa if with_map else None
        return IndexStruct(_ptr(self.req_to_token, torch.int32, "req_to_token"), self.req_to_token.shape[0],
                           self.req_to_token.shape[1], _ptr(self.req_pool_idx, torch.int32, "req_pool_idx"),
                           _ptr(self.seq_lens, torch.int32, "seq_lens"), _ptr(m, torch.int64, "full_to_swa"),
                           0 if m is None else m.numel(), self.seq_lens.numel(), self.page_size)


# ---------------------------------------------------------------------------
# entry points (same names as the C ABI)
# ---------------------------------------------------------------------------


def swa_pool_config(avail_bytes: int, ratio: float, page_size: int, window: int, n_full_layers: int,
                    full_bytes_per_token: int, n_swa_layers: int, swa_bytes_per_token: int):
    """Returns (status, n_full_tokens, n_swa_tokens); raises on argument errors
    (SWA_E_NOSPACE is returned, not raised, so callers can report the sizes)."""
    nf, ns = _i64(), _i64()
    st = lib.swa_pool_config(avail_bytes, ratio, page_size, window, n_full_layers, full_bytes_per_token, n_swa_layers,
                             swa_bytes_per_token, ctypes.byref(nf), ctypes.byref(ns))
    if st not in (SWA_OK, SWA_E_NOSPACE):
        _check(st, "swa_pool_config")
    return st, nf.value, ns.value


def swa_translate_loc(full_loc: torch.Tensor, full_to_swa: torch.Tensor, swa_loc: torch.Tensor, stream=None):
    if full_loc.numel() != swa_loc.numel():
        raise ValueError("full_loc and swa_loc must have the same length")
    _check(lib.swa_translate_loc(_ptr(full_loc, torch.int64, "full_loc"), full_loc.numel(),
                                 _ptr(full_to_swa, torch.int64, "full_to_swa"), full_to_swa.numel(),
                                 _ptr(swa_loc, torch.int64, "swa_loc"), _stream(stream)), "swa_translate_loc")


def swa_translate_window(index: IndexTables, window: int, slot_table: torch.Tensor, table_indptr: torch.Tensor,
                         prefix_lens: Optional[torch.Tensor] = None, use_map: bool = True, stream=None):
    if table_indptr.numel() < index.seq_lens.numel() + 1:
        raise ValueError("table_indptr needs batch + 1 entries")
    s = index.struct(with_map=use_map)
    _check(lib.swa_translate_window(ctypes.byref(s), window, _ptr(prefix_lens, torch.int32, "prefix_lens"),
                                    _ptr(slot_table, torch.int32, "slot_table"),
                                    _ptr(table_indptr, torch.int32, "table_indptr"), slot_table.numel(),
                                    _stream(stream)), "swa_translate_window")


def swa_kv_store(layer: KvLayer, loc: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor, stream=None):
    if k_new.shape != v_new.shape or k_new.shape[0] != loc.numel():
        raise ValueError("k_new / v_new must be (n, kv_heads, head_dim) with n = len(loc)")
    s = layer.struct()
    if k_new.numel() and tuple(k_new.shape[1:]) != (s.kv_heads, s.head_dim):
        raise ValueError("new rows must match the pool's (kv_heads, head_dim)")
    _check(lib.swa_kv_store(ctypes.byref(s), _ptr(loc, torch.int64, "loc"), loc.numel(), _ptr(k_new, name="k_new"),
                            _ptr(v_new, name="v_new"), dtype_code(k_new), _stream(stream)), "swa_kv_store")


def swa_decode_plan(batch: int, q_heads: int, kv_heads: int, head_dim: int, window: int, max_seq_len: int):
    ns, ws = _i32(), _sz()
    _check(lib.swa_decode_plan(batch, q_heads, kv_heads, head_dim, window, max_seq_len, ctypes.byref(ns),
                               ctypes.byref(ws)), "swa_decode_plan")
    return ns.value, ws.value


def swa_decode(q: torch.Tensor, layer: KvLayer, index: IndexTables, window: int, out: torch.Tensor,
               sinks: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
               slot_table: Optional[torch.Tensor] = None, table_indptr: Optional[torch.Tensor] = None,
               num_splits: int = 1, workspace: Optional[torch.Tensor] = None, use_map: bool = True, stream=None):
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be (batch, q_heads, head_dim)")
    scale = sm_scale if sm_scale is not None else q.shape[2] ** -0.5
    ls, ix = layer.struct(), index.struct(with_map=use_map)
    _check(lib.swa_decode(_ptr(q, name="q"), dtype_code(q), q.shape[1], ctypes.byref(ls), ctypes.byref(ix),
                          _ptr(slot_table, torch.int32, "slot_table"), _ptr(table_indptr, torch.int32, "table_indptr"),
                          0 if slot_table is None else slot_table.numel(), window,
                          _ptr(sinks, torch.float32, "sinks"), scale, _ptr(out, name="out"), dtype_code(out),
                          num_splits, _ptr(workspace, name="workspace"),
                          0 if workspace is None else workspace.numel() * workspace.element_size(), _stream(stream)),
           "swa_decode")


def swa_decode_noalloc(q: torch.Tensor, layer: KvLayer, index: IndexTables, window: int, out: torch.Tensor,
                       sinks: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                       slot_table: Optional[torch.Tensor] = None, table_indptr: Optional[torch.Tensor] = None,
                       num_splits: int = 1, use_map: bool = True, stream=None):
    """swa_decode with the split partials in the library's static scratch (no workspace)."""
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be (batch, q_heads, head_dim)")
    scale = sm_scale if sm_scale is not None else q.shape[2] ** -0.5
    ls, ix = layer.struct(), index.struct(with_map=use_map)
    _check(lib.swa_decode_noalloc(_ptr(q, name="q"), dtype_code(q), q.shape[1], ctypes.byref(ls), ctypes.byref(ix),
                                  _ptr(slot_table, torch.int32, "slot_table"),
                                  _ptr(table_indptr, torch.int32, "table_indptr"),
                                  0 if slot_table is None else slot_table.numel(), window,
                                  _ptr(sinks, torch.float32, "sinks"), scale, _ptr(out, name="out"), dtype_code(out),
                                  num_splits, _stream(stream)), "swa_decode_noalloc")


def swa_decode_store(q: torch.Tensor, layer: KvLayer, index: IndexTables, window: int, out: torch.Tensor,
                     loc: torch.Tensor, k_new: torch.Tensor, v_new: torch.Tensor,
                     sinks: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                     slot_table: Optional[torch.Tensor] = None, table_indptr: Optional[torch.Tensor] = None,
                     use_map: bool = True, stream=None):
    """swa_kv_store(layer, loc, k_new, v_new) then swa_decode(...) in one launch."""
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be (batch, q_heads, head_dim)")
    if k_new.shape != v_new.shape or k_new.shape[0] != loc.numel() or loc.numel() != q.shape[0]:
        raise ValueError("k_new / v_new must be (batch, kv_heads, head_dim) with one loc per request")
    ls, ix = layer.struct(), index.struct(with_map=use_map)
    if tuple(k_new.shape[1:]) != (ls.kv_heads, ls.head_dim):
        raise ValueError("new rows must match the pool's (kv_heads, head_dim)")
    scale = sm_scale if sm_scale is not None else q.shape[2] ** -0.5
    _check(lib.swa_decode_store(_ptr(q, name="q"), dtype_code(q), q.shape[1], ctypes.byref(ls), ctypes.byref(ix),
                                _ptr(slot_table, torch.int32, "slot_table"),
                                _ptr(table_indptr, torch.int32, "table_indptr"),
                                0 if slot_table is None else slot_table.numel(), window,
                                _ptr(sinks, torch.float32, "sinks"), scale, _ptr(loc, torch.int64, "loc"),
                                _ptr(k_new, name="k_new"), _ptr(v_new, name="v_new"), dtype_code(k_new),
                                _ptr(out, name="out"), dtype_code(out), _stream(stream)), "swa_decode_store")


class DecodeStep:
    """The arguments of swa_decode_step, marshalled once (the host arrays are
    kept alive here).  layers_mapping: one (pool_layer, is_swa) pair per global
    layer; q, out (and sinks, k_new, v_new when given): one tensor (or None for
    sinks) per global layer."""

    def __init__(self, layers_mapping, full_layers, swa_layers, window: int, q, out, sinks=None,
                 sm_scale: Optional[float] = None, full_loc: Optional[torch.Tensor] = None,
                 swa_loc: Optional[torch.Tensor] = None, k_new=None, v_new=None):
        n = len(layers_mapping)
        if len(q) != n or len(out) != n or (sinks is not None and len(sinks) != n):
            raise ValueError("q, out and sinks need one entry per layer")
        if (k_new is None) != (v_new is None) or (k_new is not None and (len(k_new) != n or len(v_new) != n)):
            raise ValueError("k_new and v_new need one entry per layer, or neither is given")
        self._map = (LayerMapStruct * max(n, 1))(*[LayerMapStruct(int(p), int(bool(w))) for p, w in layers_mapping])
        self._full = (KvLayerStruct * max(len(full_layers), 1))(*[ly.struct() for ly in full_layers])
        self._swa = (KvLayerStruct * max(len(swa_layers), 1))(*[ly.struct() for ly in swa_layers])
        ptrs = lambda ts, name: (ctypes.c_void_p * max(n, 1))(*[_ptr(t, name=name) for t in ts])  # noqa: E731
        self._q, self._out = ptrs(q, "q"), ptrs(out, "out")
        self._sinks = None if sinks is None else (ctypes.c_void_p * max(n, 1))(
            *[_ptr(t, torch.float32, "sinks") for t in sinks])
        self._k = None if k_new is None else ptrs(k_new, "k_new")
        self._v = None if v_new is None else ptrs(v_new, "v_new")
        self.tensors = (q, out, sinks, k_new, v_new, full_loc, swa_loc, full_layers, swa_layers)
        scale = sm_scale if sm_scale is not None else q[0].shape[2] ** -0.5
        cast = lambda a, t: None if a is None else ctypes.cast(a, ctypes.POINTER(t))  # noqa: E731
        self.struct = DecodeStepStruct(
            n, cast(self._map, LayerMapStruct), cast(self._full, KvLayerStruct), len(full_layers),
            cast(self._swa, KvLayerStruct), len(swa_layers), window, q[0].shape[1], dtype_code(q[0]),
            dtype_code(out[0]), cast(self._q, ctypes.c_void_p), cast(self._out, ctypes.c_void_p),
            cast(self._sinks, ctypes.c_void_p), scale, _ptr(full_loc, torch.int64, "full_loc"),
            _ptr(swa_loc, torch.int64, "swa_loc"), cast(self._k, ctypes.c_void_p), cast(self._v, ctypes.c_void_p))

    def workspace_bytes(self, index: IndexTables, max_seq_len: int) -> int:
        ix = index.struct()
        return lib.swa_decode_step_workspace_bytes(ctypes.byref(self.struct), ctypes.byref(ix), max_seq_len)


def swa_decode_step(step: DecodeStep, index: IndexTables, max_seq_len: int, slot_table: torch.Tensor,
                    table_indptr: torch.Tensor, workspace: Optional[torch.Tensor] = None, stream=None):
    """One decode step over every layer of a hybrid model (see swa.h)."""
    ix = index.struct()
    _check(lib.swa_decode_step(ctypes.byref(step.struct), ctypes.byref(ix), max_seq_len,
                               _ptr(slot_table, torch.int32, "slot_table"),
                               _ptr(table_indptr, torch.int32, "table_indptr"), slot_table.numel(),
                               _ptr(workspace, name="workspace"),
                               0 if workspace is None else workspace.numel() * workspace.element_size(),
                               _stream(stream)), "swa_decode_step")


def swa_extend(q: torch.Tensor, qo_indptr: torch.Tensor, prefix_lens: torch.Tensor, layer: KvLayer,
               index: IndexTables, window: int, out: torch.Tensor, sinks: Optional[torch.Tensor] = None,
               sm_scale: Optional[float] = None, slot_table: Optional[torch.Tensor] = None,
               table_indptr: Optional[torch.Tensor] = None, use_map: bool = True, stream=None):
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be (total_q, q_heads, head_dim)")
    scale = sm_scale if sm_scale is not None else q.shape[2] ** -0.5
    ls, ix = layer.struct(), index.struct(with_map=use_map)
    _check(lib.swa_extend(_ptr(q, name="q"), dtype_code(q), q.shape[1], _ptr(qo_indptr, torch.int32, "qo_indptr"),
                          _ptr(prefix_lens, torch.int32, "prefix_lens"), q.shape[0], ctypes.byref(ls),
                          ctypes.byref(ix), _ptr(slot_table, torch.int32, "slot_table"),
                          _ptr(table_indptr, torch.int32, "table_indptr"),
                          0 if slot_table is None else slot_table.numel(), window,
                          _ptr(sinks, torch.float32, "sinks"), scale, _ptr(out, name="out"), dtype_code(out),
                          _stream(stream)), "swa_extend")


def swa_validate(index: IndexTables, window: int, pool_rows: int, prefix_lens: Optional[torch.Tensor] = None,
                 store_loc: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None,
                 use_map: bool = True, qo_indptr: Optional[torch.Tensor] = None, total_q: int = 0,
                 stream=None) -> dict:
    """Counts of contract violations in the batch's index data (synchronous).
    The workspace is allocated here when not given."""
    if workspace is None:
        nbytes = lib.swa_validate_workspace_bytes(pool_rows)
        workspace = torch.empty((nbytes + 15) // 16 * 4, dtype=torch.int32, device=index.seq_lens.device)
    rep = ValidateReportStruct()
    ix = index.struct(with_map=use_map)
    _check(lib.swa_validate(ctypes.byref(ix), window, _ptr(prefix_lens, torch.int32, "prefix_lens"),
                            _ptr(qo_indptr, torch.int32, "qo_indptr"), total_q, pool_rows,
                            _ptr(store_loc, torch.int64, "store_loc"), 0 if store_loc is None else store_loc.numel(),
                            _ptr(workspace, name="workspace"), workspace.numel() * workspace.element_size(),
                            ctypes.byref(rep), _stream(stream)), "swa_validate")
    return {f: getattr(rep, f) for f in VALIDATE_FIELDS}


def swa_evict(index: IndexTables, full_to_swa: torch.Tensor, pre_lens: torch.Tensor, evicted_lens: torch.Tensor,
              window: int, freed_pages: torch.Tensor, freed_count: torch.Tensor, mode: int = 0, interval: int = 0,
              protected_lens: Optional[torch.Tensor] = None, workspace: Optional[torch.Tensor] = None, stream=None):
    """Release out-of-window SWA slots (mapping and evicted_lens updated in
    place; released pages into freed_pages, their number into freed_count)."""
    B = index.seq_lens.numel()
    if workspace is None:
        need = lib.swa_evict_workspace_bytes(B, index.req_to_token.shape[1], index.page_size)
        workspace = torch.empty(max(need // 4, 1), dtype=torch.int32, device=full_to_swa.device)
    ix = index.struct(with_map=False)
    ix.map_len = full_to_swa.numel()
    _check(lib.swa_evict(ctypes.byref(ix), _ptr(full_to_swa, torch.int64, "full_to_swa"),
                         _ptr(pre_lens, torch.int32, "pre_lens"), _ptr(protected_lens, torch.int32, "protected_lens"),
                         _ptr(evicted_lens, torch.int32, "evicted_lens"), window, mode, interval,
                         _ptr(freed_pages, torch.int64, "freed_pages"), freed_pages.numel(),
                         _ptr(freed_count, torch.int64, "freed_count"), _ptr(workspace, torch.int32, "workspace"),
                         workspace.numel() * 4, _stream(stream)), "swa_evict")


def _host_i32(a) -> Optional[np.ndarray]:
    """A host copy of lengths as a contiguous int32 numpy array (kept alive by the caller)."""
    if a is None:
        return None
    if isinstance(a, torch.Tensor):
        if a.is_cuda:
            raise ValueError("host lengths must be on the host")
        a = a.numpy()
    return np.ascontiguousarray(a, dtype=np.int32)


def _free_list(t: Optional[torch.Tensor], name: str):
    if t is None:
        return None
    return FreeListStruct(_ptr(t, torch.int64, name) if t.numel() else None, t.numel())


def swa_alloc_pages_needed(pre_lens_host, seq_lens_host, page_size: int) -> int:
    """Exact new-page count from host lengths (pre_lens_host None: decode)."""
    pre, seq = _host_i32(pre_lens_host), _host_i32(seq_lens_host)
    n = lib.swa_alloc_pages_needed(None if pre is None else pre.ctypes.data, seq.ctypes.data, seq.size, page_size)
    if n < 0:
        raise SwaError(SWA_E_ARG, "swa_alloc_pages_needed")
    return n


def swa_alloc_extend(pre_lens: torch.Tensor, seq_lens: torch.Tensor, last_loc: torch.Tensor, page_size: int,
                     free_full: torch.Tensor, out_full: torch.Tensor, free_swa: Optional[torch.Tensor] = None,
                     full_to_swa: Optional[torch.Tensor] = None, out_swa: Optional[torch.Tensor] = None,
                     new_pages: Optional[torch.Tensor] = None, pre_lens_host=None, seq_lens_host=None,
                     stream=None) -> bool:
    """Allocate the new positions [pre, seq) of every request (free lists
    passed from their heads).  Returns False, changing nothing, when the free
    lists are not provably long enough."""
    pre_h, seq_h = _host_i32(pre_lens_host), _host_i32(seq_lens_host)
    ff, fs = _free_list(free_full, "free_full"), _free_list(free_swa, "free_swa")
    if out_swa is not None and out_swa.numel() < out_full.numel():
        raise ValueError("out_swa must be as long as out_full")
    st = lib.swa_alloc_extend(seq_lens.numel(), page_size, _ptr(pre_lens, torch.int32, "pre_lens"),
                              _ptr(seq_lens, torch.int32, "seq_lens"), _ptr(last_loc, torch.int64, "last_loc"),
                              ctypes.byref(ff), None if fs is None else ctypes.byref(fs),
                              _ptr(full_to_swa, torch.int64, "full_to_swa"),
                              0 if full_to_swa is None else full_to_swa.numel(), out_full.numel(),
                              None if pre_h is None else pre_h.ctypes.data,
                              None if seq_h is None else seq_h.ctypes.data, _ptr(out_full, torch.int64, "out_full"),
                              _ptr(out_swa, torch.int64, "out_swa"), _ptr(new_pages, torch.int64, "new_pages"),
                              _stream(stream))
    if st == SWA_E_NOSPACE:
        return False
    _check(st, "swa_alloc_extend")
    return True


def swa_alloc_decode(seq_lens: torch.Tensor, last_loc: torch.Tensor, page_size: int, free_full: torch.Tensor,
                     out_full: torch.Tensor, free_swa: Optional[torch.Tensor] = None,
                     full_to_swa: Optional[torch.Tensor] = None, out_swa: Optional[torch.Tensor] = None,
                     new_pages: Optional[torch.Tensor] = None, seq_lens_host=None, stream=None) -> bool:
    """One new token per request; returns False, changing nothing, when the
    free lists are not provably long enough."""
    seq_h = _host_i32(seq_lens_host)
    ff, fs = _free_list(free_full, "free_full"), _free_list(free_swa, "free_swa")
    if out_full.numel() < seq_lens.numel() or (out_swa is not None and out_swa.numel() < seq_lens.numel()):
        raise ValueError("out_full and out_swa need one entry per request")
    st = lib.swa_alloc_decode(seq_lens.numel(), page_size, _ptr(seq_lens, torch.int32, "seq_lens"),
                              _ptr(last_loc, torch.int64, "last_loc"), ctypes.byref(ff),
                              None if fs is None else ctypes.byref(fs), _ptr(full_to_swa, torch.int64, "full_to_swa"),
                              0 if full_to_swa is None else full_to_swa.numel(),
                              None if seq_h is None else seq_h.ctypes.data, _ptr(out_full, torch.int64, "out_full"),
                              _ptr(out_swa, torch.int64, "out_swa"), _ptr(new_pages, torch.int64, "new_pages"),
                              _stream(stream))
    if st == SWA_E_NOSPACE:
        return False
    _check(st, "swa_alloc_decode")
    return True


# ---------------------------------------------------------------------------
# unified pool
# ---------------------------------------------------------------------------

_DTYPE_CODE = {torch.float32: SWA_F32, torch.bfloat16: SWA_BF16, torch.uint8: SWA_FP8_E4M3,
               torch.float8_e4m3fn: SWA_FP8_E4M3}


def swa_unified_pool_bytes(layer_num: int, kv_heads: int, head_dim: int, dtype: torch.dtype, page_size: int,
                           num_pages: int) -> int:
    n = lib.swa_unified_pool_bytes(layer_num, kv_heads, head_dim, _DTYPE_CODE[dtype], page_size, num_pages)
    if n < 0:
        raise SwaError(SWA_E_ARG, "swa_unified_pool_bytes")
    return n


@dataclass
class RawKvLayer:
    """A layer view the library computed over a raw buffer (kept alive here)."""
    raw: torch.Tensor
    view: KvLayerStruct

    def struct(self) -> KvLayerStruct:
        return self.view


def swa_unified_layer_views(raw: torch.Tensor, anchor_bytes: int, layer_num: int, kv_heads: int, head_dim: int,
                            dtype: torch.dtype, page_size: int, num_pages: int, k_scale: float = 1.0,
                            v_scale: float = 1.0):
    """Per-layer K/V views of a unified sub-pool in `raw` (a uint8 device tensor)."""
    views = (KvLayerStruct * layer_num)()
    _check(lib.swa_unified_layer_views(_ptr(raw, torch.uint8, "raw"), raw.numel(), anchor_bytes, layer_num, kv_heads,
                                       head_dim, _DTYPE_CODE[dtype], page_size, num_pages, k_scale, v_scale, views),
           "swa_unified_layer_views")
    return [RawKvLayer(raw, KvLayerStruct(v.k, v.v, v.rows, v.kv_heads, v.head_dim, v.dtype, v.k_scale, v.v_scale))
            for v in views]


def swa_translate_kernel_ids(virt: torch.Tensor, v2p: torch.Tensor, page_size: int, multiplier: int,
                             out: torch.Tensor, stream=None):
    if virt.numel() != out.numel():
        raise ValueError("virt and out must have the same length")
    _check(lib.swa_translate_kernel_ids(_ptr(virt, torch.int64, "virt"), virt.numel(), _ptr(v2p, torch.int64, "v2p"),
                                        v2p.numel(), page_size, multiplier, _ptr(out, torch.int64, "out"),
                                        _stream(stream)), "swa_translate_kernel_ids")


def swa_translate_window_unified(index: IndexTables, v2p: torch.Tensor, multiplier: int, window: int,
                                 slot_table: torch.Tensor, table_indptr: torch.Tensor,
                                 prefix_lens: Optional[torch.Tensor] = None, stream=None):
    if table_indptr.numel() < index.seq_lens.numel() + 1:
        raise ValueError("table_indptr needs batch + 1 entries")
    ix = index.struct(with_map=False)
    _check(lib.swa_translate_window_unified(ctypes.byref(ix), _ptr(v2p, torch.int64, "v2p"), v2p.numel(), multiplier,
                                            window, _ptr(prefix_lens, torch.int32, "prefix_lens"),
                                            _ptr(slot_table, torch.int32, "slot_table"),
                                            _ptr(table_indptr, torch.int32, "table_indptr"), slot_table.numel(),
                                            _stream(stream)), "swa_translate_window_unified")


# ---------------------------------------------------------------------------
# attention variants: chunked local attention, per-request SWA ring
# ---------------------------------------------------------------------------


def swa_translate_window_chunked(index: IndexTables, window: int, chunk: int, slot_table: torch.Tensor,
                                 table_indptr: torch.Tensor, prefix_lens: Optional[torch.Tensor] = None,
                                 use_map: bool = True, stream=None):
    if table_indptr.numel() < index.seq_lens.numel() + 1:
        raise ValueError("table_indptr needs batch + 1 entries")
    ix = index.struct(with_map=use_map)
    _check(lib.swa_translate_window_chunked(ctypes.byref(ix), window, chunk,
                                            _ptr(prefix_lens, torch.int32, "prefix_lens"),
                                            _ptr(slot_table, torch.int32, "slot_table"),
                                            _ptr(table_indptr, torch.int32, "table_indptr"), slot_table.numel(),
                                            _stream(stream)), "swa_translate_window_chunked")


def swa_extend_chunked(q: torch.Tensor, qo_indptr: torch.Tensor, prefix_lens: torch.Tensor, layer: KvLayer,
                       index: IndexTables, window: int, chunk: int, out: torch.Tensor,
                       sinks: Optional[torch.Tensor] = None, sm_scale: Optional[float] = None,
                       slot_table: Optional[torch.Tensor] = None, table_indptr: Optional[torch.Tensor] = None,
                       use_map: bool = True, stream=None):
    if q.dim() != 3 or out.shape != q.shape:
        raise ValueError("q and out must be (total_q, q_heads, head_dim)")
    scale = sm_scale if sm_scale is not None else q.shape[2] ** -0.5
    ls, ix = layer.struct(), index.struct(with_map=use_map)
    _check(lib.swa_extend_chunked(_ptr(q, name="q"), dtype_code(q), q.shape[1],
                                  _ptr(qo_indptr, torch.int32, "qo_indptr"), _ptr(prefix_lens, torch.int32, "prefix_lens"),
                                  q.shape[0], ctypes.byref(ls), ctypes.byref(ix),
                                  _ptr(slot_table, torch.int32, "slot_table"),
                                  _ptr(table_indptr, torch.int32, "table_indptr"),
                                  0 if slot_table is None else slot_table.numel(), window, chunk,
                                  _ptr(sinks, torch.float32, "sinks"), scale, _ptr(out, name="out"), dtype_code(out),
                                  _stream(stream)), "swa_extend_chunked")


def _ring_index(req_pool_idx: torch.Tensor, seq_lens: torch.Tensor, request_slots: int, max_len: int) -> IndexStruct:
    return IndexStruct(None, request_slots, max_len, _ptr(req_pool_idx, torch.int32, "req_pool_idx"),
                       _ptr(seq_lens, torch.int32, "seq_lens"), None, 0, seq_lens.numel(), 1)


def swa_translate_window_ring(req_pool_idx: torch.Tensor, seq_lens: torch.Tensor, request_slots: int, max_len: int,
                              ring_rows: int, window: int, slot_table: torch.Tensor, table_indptr: torch.Tensor,
                              chunk: int = 0, prefix_lens: Optional[torch.Tensor] = None, stream=None):
    """Window slot table of a per-request SWA ring (request slot r, position j
    -> r * ring_rows + j mod ring_rows)."""
    if table_indptr.numel() < seq_lens.numel() + 1:
        raise ValueError("table_indptr needs batch + 1 entries")
    ix = _ring_index(req_pool_idx, seq_lens, request_slots, max_len)
    _check(lib.swa_translate_window_ring(ctypes.byref(ix), ring_rows, window, chunk,
                                         _ptr(prefix_lens, torch.int32, "prefix_lens"),
                                         _ptr(slot_table, torch.int32, "slot_table"),
                                         _ptr(table_indptr, torch.int32, "table_indptr"), slot_table.numel(),
                                         _stream(stream)), "swa_translate_window_ring")


def swa_ring_locs(req_pool_idx: torch.Tensor, seq_lens: torch.Tensor, request_slots: int, ring_rows: int,
                  out: torch.Tensor, prefix_lens: Optional[torch.Tensor] = None, stream=None):
    """Ring rows of the new positions (prefix_lens None: one decode position
    per request)."""
    ix = _ring_index(req_pool_idx, seq_lens, request_slots, 1)
    _check(lib.swa_ring_locs(ctypes.byref(ix), ring_rows, _ptr(prefix_lens, torch.int32, "prefix_lens"),
                             _ptr(out, torch.int64, "out"), out.numel(), _stream(stream)), "swa_ring_locs")


def swa_probe_read(buf: torch.Tensor, out: torch.Tensor, grid: int, stream=None):
    """One streaming read of `buf` (16-aligned, a multiple of 16 bytes); out holds grid * 256 floats."""
    if out.numel() < grid * 256:
        raise ValueError("out needs grid * 256 floats")
    _check(lib.swa_probe_read(_ptr(buf, name="buf"), buf.numel() * buf.element_size(),
                              _ptr(out, torch.float32, "out"), grid, _stream(stream)), "swa_probe_read")


def swa_probe_copy(src: torch.Tensor, dst: torch.Tensor, grid: int, stream=None):
    """One copy of src into dst (same byte size, 16-aligned, not overlapping)."""
    nbytes = src.numel() * src.element_size()
    if dst.numel() * dst.element_size() != nbytes:
        raise ValueError("src and dst must have the same size in bytes")
    _check(lib.swa_probe_copy(_ptr(src, name="src"), _ptr(dst, name="dst"), nbytes, grid, _stream(stream)),
           "swa_probe_copy")


def swa_probe_mfma(out: torch.Tensor, grid: int, iters: int, stream=None):
    """grid * 4 * iters * 8 bf16 MFMAs of 16,384 FLOPs; out holds grid * 256 floats."""
    if out.numel() < grid * 256:
        raise ValueError("out needs grid * 256 floats")
    _check(lib.swa_probe_mfma(_ptr(out, torch.float32, "out"), grid, iters, _stream(stream)), "swa_probe_mfma")
