"""Python binding of libswr: sharded weight reassembly on one MI355X (gfx950).

Argument marshalling only.  Every step of the path runs in the HIP library
(``libswr.so``, built in-tree by ``sharded_weight_reassembly_amd.build``);
PyTorch supplies device memory and streams.  The functions carry the names
of the C entry points in ``include/swr.h`` without the ``swr_`` prefix.

If the library has not been built, importing the binding's functions raises
ImportError: there is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
from typing import Sequence

import torch  # loaded first: libswr binds to the HIP runtime torch has loaded

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libswr.so")

BF16 = 0
FP8_E4M3FN = 1
DTYPES = {"bf16": BF16, "fp8_e4m3fn": FP8_E4M3FN}
ELEM_BYTES = {BF16: 2, FP8_E4M3FN: 1}

OK, E_INVALID, E_ALIGN, E_CAPACITY, E_SHAPE, E_HIP, E_SEQUENCE = 0, -1, -2, -3, -4, -5, -6
STATUS_NAMES = {0: "SWR_OK", -1: "SWR_E_INVALID", -2: "SWR_E_ALIGN", -3: "SWR_E_CAPACITY", -4: "SWR_E_SHAPE",
                -5: "SWR_E_HIP", -6: "SWR_E_SEQUENCE"}

TRACE_OPS = {1: "record_start", 2: "wait_start", 3: "wait_done", 4: "copy", 5: "record_ready", 6: "wait_ready",
             7: "record_done", 8: "copy_next", 9: "record_begin", 10: "wait_begin", 11: "record_free",
             12: "wait_free"}
TRACE_STREAMS = {0: "compute", 1: "side", 2: "prefetch"}

# Every function include/swr.h declares.
EXPORTS = (
    "swr_plan_layer", "swr_pack_layer", "swr_redistribute_row_shards", "swr_reassemble_into_slot",
    "swr_reassemble_into_slot_dma",
    "swr_planner_set_copy_engine", "swr_planner_set_gate", "swr_planner_set_gather_lds", "swr_proj_forward",
    "swr_proj_workspace_bytes", "swr_proj_forward_grouped", "swr_proj_grouped_workspace_bytes", "swr_mlp_forward",
    "swr_mlp_forward_partial", "swr_mlp_workspace_bytes", "swr_mlp_forward_noalloc", "swr_sum_partials",
    "swr_quantize_rows_e4m3",
    "swr_mlp_forward_fp8act", "swr_mlp_fp8act_workspace_bytes",
    "swr_planner_create", "swr_planner_set_layer", "swr_planner_reset", "swr_planner_pre_dispatch",
    "swr_planner_maybe_dispatch", "swr_planner_wait_ready_once", "swr_planner_update_done_event",
    "swr_planner_counters", "swr_planner_trace", "swr_planner_destroy", "swr_planner_set_timing",
    "swr_planner_pause_timing",
    "swr_planner_gather_times", "swr_planner_layer_times", "swr_planner_set_cyclic", "swr_planner_set_first_prefetch",
    "swr_planner_prefetch_first", "swr_last_error", "swr_version",
)


class SwrError(RuntimeError):
    def __init__(self, fn: str, code: int, message: str):
        super().__init__(f"{fn} failed with {STATUS_NAMES.get(code, code)}: {message}")
        self.code = code
        self.fn = fn


class WeightDesc(ctypes.Structure):
    _fields_ = [("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("reserved", ctypes.c_int32)]


class ViewDesc(ctypes.Structure):
    _fields_ = [("offset", ctypes.c_int64), ("nbytes", ctypes.c_int64), ("out_features", ctypes.c_int64),
                ("in_features", ctypes.c_int64), ("dtype", ctypes.c_int32), ("reserved", ctypes.c_int32)]


class Layout(ctypes.Structure):
    _fields_ = [("payload_bytes", ctypes.c_int64), ("total_bytes", ctypes.c_int64), ("chunk_bytes", ctypes.c_int64),
                ("n_weights", ctypes.c_int32), ("n_chunks", ctypes.c_int32)]


MAX_CHUNKS, MAX_SUB = 64, 4


class RowShards(ctypes.Structure):
    _fields_ = [("n_sub", ctypes.c_int32), ("replicated", ctypes.c_int32), ("sub_rows", ctypes.c_int64 * MAX_SUB),
                ("src", ctypes.c_void_p * MAX_CHUNKS)]


class ProjDesc(ctypes.Structure):
    _fields_ = [("W", ctypes.c_void_p), ("row_scale", ctypes.c_void_p), ("X", ctypes.c_void_p),
                ("Y", ctypes.c_void_p), ("out_features", ctypes.c_int64), ("in_features", ctypes.c_int64),
                ("ldx", ctypes.c_int64), ("ldy", ctypes.c_int64), ("dtype", ctypes.c_int32),
                ("y_fp32", ctypes.c_int32)]


_lib = None
_vp = ctypes.c_void_p
_i32, _i64 = ctypes.c_int32, ctypes.c_int64


def lib() -> ctypes.CDLL:
    """The loaded library; raises ImportError if it was never built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise ImportError(f"{LIB_PATH} is missing: build it with `python -m sharded_weight_reassembly_amd.build`")
    L = ctypes.CDLL(LIB_PATH)
    sig = {
        "swr_plan_layer": (_i32, [ctypes.POINTER(WeightDesc), _i32, _i32, ctypes.POINTER(ViewDesc),
                                  ctypes.POINTER(Layout)]),
        "swr_pack_layer": (_i32, [ctypes.POINTER(Layout), ctypes.POINTER(ViewDesc), ctypes.POINTER(_vp),
                                  ctypes.POINTER(_vp), _vp]),
        "swr_reassemble_into_slot": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _vp, _i64, _i32, _vp, _vp, _vp,
                                            ctypes.POINTER(_i64)]),
        "swr_redistribute_row_shards": (_i32, [ctypes.POINTER(Layout), ctypes.POINTER(ViewDesc),
                                               ctypes.POINTER(RowShards), ctypes.POINTER(_vp), _vp]),
        "swr_reassemble_into_slot_dma": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _vp, _i64, _i32, _vp, _vp, _vp,
                                                ctypes.POINTER(_i64)]),
        "swr_planner_set_copy_engine": (_i32, [_vp, _i32]),
        "swr_planner_set_gate": (_i32, [_vp, _i32]),
        "swr_planner_set_gather_lds": (_i32, [_vp, _i32]),
        "swr_proj_forward": (_i32, [_vp, _i32, _vp, _i64, _i64, _vp, _i64, _i64, _vp, _i32, _i64, _vp, _i64, _vp]),
        "swr_proj_workspace_bytes": (_i64, [_i64, _i64, _i64, _i32]),
        "swr_proj_forward_grouped": (_i32, [ctypes.POINTER(ProjDesc), _i32, _i64, _vp, _i64, _vp]),
        "swr_proj_grouped_workspace_bytes": (_i64, [ctypes.POINTER(ProjDesc), _i32, _i64]),
        "swr_mlp_forward": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp]),
        "swr_mlp_workspace_bytes": (_i64, [_i64, _i64, _i64, _i32]),
        "swr_mlp_forward_noalloc": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _vp, _vp]),
        "swr_mlp_forward_partial": (_i32, [_vp, _vp, _vp, _vp, _i32, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp]),
        "swr_sum_partials": (_i32, [ctypes.POINTER(_vp), _i32, _i64, _vp, _i32, _vp]),
        "swr_quantize_rows_e4m3": (_i32, [_vp, _i64, _i64, _i64, _vp, _i64, _vp, _vp]),
        "swr_mlp_forward_fp8act": (_i32, [_vp, _vp, _vp, _vp, _i64, _i64, _vp, _i64, _vp, _vp, _i64, _vp]),
        "swr_mlp_fp8act_workspace_bytes": (_i64, [_i64, _i64, _i64]),
        "swr_planner_create": (_i32, [_i32, _i32, _vp, _vp, _vp, _vp, _i64, ctypes.POINTER(_vp)]),
        "swr_planner_set_layer": (_i32, [_vp, _i32, ctypes.POINTER(_vp), _i32, _i64]),
        "swr_planner_reset": (_i32, [_vp]),
        "swr_planner_pre_dispatch": (_i32, [_vp, _i32]),
        "swr_planner_maybe_dispatch": (_i32, [_vp, _i32]),
        "swr_planner_wait_ready_once": (_i32, [_vp, _i32, ctypes.POINTER(_vp)]),
        "swr_planner_update_done_event": (_i32, [_vp, _i32]),
        "swr_planner_counters": (_i32, [_vp, ctypes.POINTER(_i64), ctypes.POINTER(_i64)]),
        "swr_planner_trace": (_i32, [_vp, ctypes.POINTER(_i32), _i32, ctypes.POINTER(_i32)]),
        "swr_planner_destroy": (None, [_vp]),
        "swr_planner_set_timing": (_i32, [_vp, _i32]),
        "swr_planner_pause_timing": (_i32, [_vp, _i32]),
        "swr_planner_set_cyclic": (_i32, [_vp, _i32]),
        "swr_planner_set_first_prefetch": (_i32, [_vp, _vp]),
        "swr_planner_prefetch_first": (_i32, [_vp]),
        "swr_planner_gather_times": (_i32, [_vp, ctypes.POINTER(ctypes.c_float), _i32, ctypes.POINTER(_i32)]),
        "swr_planner_layer_times": (_i32, [_vp, ctypes.POINTER(ctypes.c_float), _i32, ctypes.POINTER(_i32)]),
        "swr_last_error": (ctypes.c_char_p, []),
        "swr_version": (ctypes.c_char_p, []),
    }
    for name, (res, args) in sig.items():
        f = getattr(L, name)
        f.restype = res
        f.argtypes = args
    _lib = L
    return L


def _check(fn: str, rc: int) -> int:
    if rc < 0:
        raise SwrError(fn, rc, lib().swr_last_error().decode())
    return rc


def _ptr(x) -> int | None:
    """Device address of a tensor (or an int address, or None)."""
    if x is None:
        return None
    if isinstance(x, int):
        return x
    if isinstance(x, torch.Tensor):
        if not x.is_cuda:
            raise ValueError("expected a device tensor")
        return x.data_ptr()
    raise TypeError(f"cannot take a device address of {type(x)!r}")


def _stream(s) -> int | None:
    if s is None:
        return torch.cuda.current_stream().cuda_stream
    if isinstance(s, int):
        return s
    return s.cuda_stream


def _event(e) -> int | None:
    if e is None or isinstance(e, int):
        return e
    return e.cuda_event


def _ptr_array(items) -> ctypes.Array:
    arr = (_vp * len(items))()
    for i, t in enumerate(items):
        arr[i] = _ptr(t)
    return arr


def _dtype(d) -> int:
    return DTYPES[d] if isinstance(d, str) else int(d)


# --------------------------------------------------------------- flat layout

def plan_layer(weights: Sequence[tuple[int, int, object]], n_chunks: int) -> tuple[list[dict], dict]:
    """[(out, in, dtype)] -> (views, layout); dtype is "bf16"/"fp8_e4m3fn" or its code."""
    n = len(weights)
    descs = (WeightDesc * max(n, 1))()
    for i, (o, k, d) in enumerate(weights):
        descs[i] = WeightDesc(int(o), int(k), _dtype(d), 0)
    views = (ViewDesc * max(n, 1))()
    lay = Layout()
    _check("swr_plan_layer", lib().swr_plan_layer(descs, n, int(n_chunks), views, ctypes.byref(lay)))
    vs = [dict(offset=v.offset, nbytes=v.nbytes, out_features=v.out_features, in_features=v.in_features,
               dtype=v.dtype) for v in views[:n]]
    layout = dict(payload_bytes=lay.payload_bytes, total_bytes=lay.total_bytes, chunk_bytes=lay.chunk_bytes,
                  n_weights=lay.n_weights, n_chunks=lay.n_chunks)
    return vs, layout


def _layout_struct(layout: dict) -> Layout:
    return Layout(layout["payload_bytes"], layout["total_bytes"], layout["chunk_bytes"], layout["n_weights"],
                  layout["n_chunks"])


def _views_struct(views: list[dict]) -> ctypes.Array:
    arr = (ViewDesc * max(len(views), 1))()
    for i, v in enumerate(views):
        arr[i] = ViewDesc(v["offset"], v["nbytes"], v["out_features"], v["in_features"], v["dtype"], 0)
    return arr


def pack_layer(layout: dict, views: list[dict], src, chunks, stream=None) -> None:
    """Write T (weights + zero padding) into the N chunk buffers."""
    lay = _layout_struct(layout)
    _check("swr_pack_layer", lib().swr_pack_layer(ctypes.byref(lay), _views_struct(views), _ptr_array(src),
                                                  _ptr_array(chunks), _stream(stream)))


def row_shards_struct(shards) -> ctypes.Array:
    """shards[j]: dict with "src" (list of device tensors/addresses) and either
    "replicated": True (src[0] is the whole weight) or "sub_rows"."""
    arr = (RowShards * len(shards))()
    for j, sh in enumerate(shards):
        d = arr[j]
        d.replicated = int(bool(sh.get("replicated", False)))
        rows = list(sh.get("sub_rows", []))
        d.n_sub = len(rows)
        for b, r in enumerate(rows):
            d.sub_rows[b] = int(r)
        for r, t in enumerate(sh["src"]):
            d.src[r] = _ptr(t)
    return arr


def redistribute_row_shards(layout: dict, views: list[dict], shards, chunks, stream=None) -> None:
    """Flat chunks from every weight's row shards (the loader's one-time re-layout)."""
    _check("swr_redistribute_row_shards",
           lib().swr_redistribute_row_shards(ctypes.byref(_layout_struct(layout)), _views_struct(views),
                                             row_shards_struct(shards), _ptr_array(chunks), _stream(stream)))


def reassemble_into_slot(chunks, chunk_bytes: int, slot, slot_bytes: int | None = None, self_rank: int = 0,
                         stream=None, gate=None, ready=None) -> int:
    """Gather the N chunks into `slot`; returns the bytes counted as received from peers."""
    if slot_bytes is None:
        slot_bytes = slot.numel() * slot.element_size()
    remote = _i64(0)
    _check("swr_reassemble_into_slot",
           lib().swr_reassemble_into_slot(_ptr_array(chunks), len(chunks), int(chunk_bytes), _ptr(slot),
                                          int(slot_bytes), int(self_rank), _stream(stream), _event(gate),
                                          _event(ready), ctypes.byref(remote)))
    return remote.value


def reassemble_into_slot_dma(chunks, chunk_bytes: int, slot, slot_bytes: int | None = None, self_rank: int = 0,
                             stream=None, gate=None, ready=None) -> int:
    """reassemble_into_slot on the DMA engines (no compute units)."""
    if slot_bytes is None:
        slot_bytes = slot.numel() * slot.element_size()
    remote = _i64(0)
    _check("swr_reassemble_into_slot_dma",
           lib().swr_reassemble_into_slot_dma(_ptr_array(chunks), len(chunks), int(chunk_bytes), _ptr(slot),
                                              int(slot_bytes), int(self_rank), _stream(stream), _event(gate),
                                              _event(ready), ctypes.byref(remote)))
    return remote.value


ENGINE_KERNEL, ENGINE_DMA = 0, 1
GATE_DONE, GATE_BEGIN, GATE_AFTER = 0, 1, 2


def view(slot: torch.Tensor, v: dict) -> torch.Tensor:
    """Zero-copy view of weight v inside a uint8 slot tensor (narrow + view)."""
    raw = slot.narrow(0, v["offset"], v["nbytes"])
    if v["dtype"] == BF16:
        return raw.view(torch.bfloat16).view(v["out_features"], v["in_features"])
    return raw.view(v["out_features"], v["in_features"])


# --------------------------------------------------------------------- GEMMs

def proj_workspace_bytes(m: int, out_f: int, in_f: int, dtype) -> int:
    return _check("swr_proj_workspace_bytes", lib().swr_proj_workspace_bytes(m, out_f, in_f, _dtype(dtype)))


def proj_forward(w, dtype, row_scale, out_f: int, in_f: int, x: torch.Tensor, y: torch.Tensor, m: int | None = None,
                 ldx: int | None = None, ldy: int | None = None, y_fp32: bool | None = None, workspace=None,
                 workspace_bytes: int | None = None, stream=None) -> None:
    """Y[m, o] = s[o] * sum_k X[m, k] W[o, k]; `w` is a tensor or a device address (a view)."""
    if m is None:
        m = x.shape[0]
    if ldx is None:
        ldx = x.stride(0) if x.dim() == 2 else in_f
    if ldy is None:
        ldy = y.stride(0) if y.dim() == 2 else out_f
    if y_fp32 is None:
        y_fp32 = y.dtype == torch.float32
    if workspace is not None and workspace_bytes is None:
        workspace_bytes = workspace.numel() * workspace.element_size()
    _check("swr_proj_forward",
           lib().swr_proj_forward(_ptr(w), _dtype(dtype), _ptr(row_scale), int(out_f), int(in_f), _ptr(x), int(ldx),
                                  int(m), _ptr(y), int(bool(y_fp32)), int(ldy), _ptr(workspace),
                                  int(workspace_bytes or 0), _stream(stream)))


def _proj_descs(projs) -> ctypes.Array:
    """projs: dicts with w, dtype, row_scale, out_f, in_f, x, y and optional ldx, ldy, y_fp32."""
    arr = (ProjDesc * len(projs))()
    for i, p in enumerate(projs):
        x, y = p["x"], p["y"]
        d = arr[i]
        d.W, d.row_scale, d.X, d.Y = _ptr(p["w"]), _ptr(p.get("row_scale")), _ptr(x), _ptr(y)
        d.out_features, d.in_features = int(p["out_f"]), int(p["in_f"])
        d.ldx = int(p["ldx"]) if p.get("ldx") is not None else (x.stride(0) if isinstance(x, torch.Tensor) else
                                                                  int(p["in_f"]))
        d.ldy = int(p["ldy"]) if p.get("ldy") is not None else (y.stride(0) if isinstance(y, torch.Tensor) else
                                                                  int(p["out_f"]))
        y_fp32 = p.get("y_fp32")
        if y_fp32 is None:
            y_fp32 = isinstance(y, torch.Tensor) and y.dtype == torch.float32
        d.dtype, d.y_fp32 = _dtype(p["dtype"]), int(bool(y_fp32))
    return arr


def proj_grouped_workspace_bytes(projs, m: int) -> int:
    return _check("swr_proj_grouped_workspace_bytes",
                  lib().swr_proj_grouped_workspace_bytes(_proj_descs(projs), len(projs), int(m)))


def proj_forward_grouped(projs, m: int, workspace=None, stream=None) -> None:
    """Every projection of `projs` as proj_forward would compute it, one launch where possible."""
    nb = workspace.numel() * workspace.element_size() if workspace is not None else 0
    _check("swr_proj_forward_grouped",
           lib().swr_proj_forward_grouped(_proj_descs(projs), len(projs), int(m), _ptr(workspace), nb,
                                          _stream(stream)))


def mlp_workspace_bytes(m: int, hidden: int, inter: int, dtype) -> int:
    return _check("swr_mlp_workspace_bytes", lib().swr_mlp_workspace_bytes(m, hidden, inter, _dtype(dtype)))


def mlp_forward(w_gate_up, s_gu, w_down, s_d, dtype, hidden: int, inter: int, x: torch.Tensor, y: torch.Tensor,
                workspace: torch.Tensor, m: int | None = None, stream=None) -> None:
    """Y = bf16((bf16(silu(G[:, :I]) * G[:, I:]) @ W_down^T) * s_d),  G = X @ W_gate_up^T * s_gu."""
    if m is None:
        m = x.shape[0]
    _check("swr_mlp_forward",
           lib().swr_mlp_forward(_ptr(w_gate_up), _ptr(s_gu), _ptr(w_down), _ptr(s_d), _dtype(dtype), int(hidden),
                                 int(inter), _ptr(x), int(m), _ptr(y), _ptr(workspace),
                                 workspace.numel() * workspace.element_size(), _stream(stream)))


NOALLOC_SCRATCH_BYTES = 16 << 20


def mlp_forward_noalloc(w_gate_up, s_gu, w_down, s_d, dtype, hidden: int, inter: int, x, y, m: int | None = None,
                        stream=None) -> None:
    """mlp_forward without a workspace: the library's fixed per-GPU scratch
    (NOALLOC_SCRATCH_BYTES) holds h and the split-K partials."""
    if m is None:
        m = x.shape[0]
    _check("swr_mlp_forward_noalloc",
           lib().swr_mlp_forward_noalloc(_ptr(w_gate_up), _ptr(s_gu), _ptr(w_down), _ptr(s_d), _dtype(dtype),
                                         int(hidden), int(inter), _ptr(x), int(m), _ptr(y), _stream(stream)))


def mlp_forward_partial(w_gate_up, s_gu, w_down, s_d, dtype, hidden: int, inter: int, x: torch.Tensor,
                        y: torch.Tensor, workspace: torch.Tensor, m: int | None = None, stream=None) -> None:
    """One rank's fp32 partial of the MLP over its intermediate slice (no rounding of Y)."""
    if m is None:
        m = x.shape[0]
    _check("swr_mlp_forward_partial",
           lib().swr_mlp_forward_partial(_ptr(w_gate_up), _ptr(s_gu), _ptr(w_down), _ptr(s_d), _dtype(dtype),
                                         int(hidden), int(inter), _ptr(x), int(m), _ptr(y), _ptr(workspace),
                                         workspace.numel() * workspace.element_size(), _stream(stream)))


def quantize_rows_e4m3(x: torch.Tensor, q: torch.Tensor, s: torch.Tensor, m: int | None = None,
                       stream=None) -> None:
    """Per-token E4M3FN codes q [M, K] (uint8) and scales s [M] (fp32) of bf16 rows x [M, K]."""
    if m is None:
        m = x.shape[0]
    k = x.shape[1]
    _check("swr_quantize_rows_e4m3", lib().swr_quantize_rows_e4m3(_ptr(x), x.stride(0), int(m), int(k), _ptr(q),
                                                                  q.stride(0), _ptr(s), _stream(stream)))


def mlp_fp8act_workspace_bytes(m: int, hidden: int, inter: int) -> int:
    return _check("swr_mlp_fp8act_workspace_bytes", lib().swr_mlp_fp8act_workspace_bytes(m, hidden, inter))


def mlp_forward_fp8act(w_gate_up, s_gu, w_down, s_d, hidden: int, inter: int, x: torch.Tensor, y: torch.Tensor,
                       workspace: torch.Tensor, m: int | None = None, stream=None) -> None:
    """The MLP with FP8 weights and per-token FP8 activations (X and h quantised)."""
    if m is None:
        m = x.shape[0]
    _check("swr_mlp_forward_fp8act",
           lib().swr_mlp_forward_fp8act(_ptr(w_gate_up), _ptr(s_gu), _ptr(w_down), _ptr(s_d), int(hidden), int(inter),
                                        _ptr(x), int(m), _ptr(y), _ptr(workspace),
                                        workspace.numel() * workspace.element_size(), _stream(stream)))


def sum_partials(parts, out: torch.Tensor, count: int | None = None, stream=None) -> None:
    """out = parts[0] + ... + parts[n-1] (fp32, in order); out fp32 or bf16."""
    if count is None:
        count = out.numel()
    _check("swr_sum_partials", lib().swr_sum_partials(_ptr_array(parts), len(parts), int(count), _ptr(out),
                                                      int(out.dtype == torch.bfloat16), _stream(stream)))


# ------------------------------------------------------------------ planner

class Planner:
    """Lookahead / ping-pong scheduler over layers [start, end) (owns its events)."""

    def __init__(self, start: int, end: int, compute, side, slot_a: torch.Tensor, slot_b: torch.Tensor,
                 slot_bytes: int | None = None):
        if slot_bytes is None:
            slot_bytes = min(slot_a.numel() * slot_a.element_size(), slot_b.numel() * slot_b.element_size())
        h = _vp()
        _check("swr_planner_create", lib().swr_planner_create(int(start), int(end), _stream(compute), _stream(side),
                                                              _ptr(slot_a), _ptr(slot_b), int(slot_bytes),
                                                              ctypes.byref(h)))
        self._h = h
        self.start, self.end = start, end
        self._keep = (slot_a, slot_b)

    def set_layer(self, layer: int, chunks, chunk_bytes: int) -> None:
        _check("swr_planner_set_layer", lib().swr_planner_set_layer(self._h, int(layer), _ptr_array(chunks),
                                                                    len(chunks), int(chunk_bytes)))

    def reset(self) -> None:
        _check("swr_planner_reset", lib().swr_planner_reset(self._h))

    def pre_dispatch(self, layer: int) -> None:
        _check("swr_planner_pre_dispatch", lib().swr_planner_pre_dispatch(self._h, int(layer)))

    def maybe_dispatch(self, layer: int) -> None:
        _check("swr_planner_maybe_dispatch", lib().swr_planner_maybe_dispatch(self._h, int(layer)))

    def wait_ready_once(self, layer: int) -> int:
        out = _vp()
        _check("swr_planner_wait_ready_once", lib().swr_planner_wait_ready_once(self._h, int(layer), ctypes.byref(out)))
        return out.value

    def update_done_event(self, layer: int) -> None:
        _check("swr_planner_update_done_event", lib().swr_planner_update_done_event(self._h, int(layer)))

    def set_cyclic(self, enabled: bool) -> None:
        """Gather the next forward's first layer during the last layer (even layer counts)."""
        _check("swr_planner_set_cyclic", lib().swr_planner_set_cyclic(self._h, int(bool(enabled))))

    def set_first_prefetch(self, stream) -> None:
        """Gather the first layer on a dedicated stream (None: off); see prefetch_first."""
        _check("swr_planner_set_first_prefetch",
               lib().swr_planner_set_first_prefetch(self._h, None if stream is None else _stream(stream)))

    def prefetch_first(self) -> None:
        """On the dedicated stream: wait for slot 0 to be free, gather the first layer, record its ready event."""
        _check("swr_planner_prefetch_first", lib().swr_planner_prefetch_first(self._h))

    def set_gate(self, gate: int) -> None:
        """GATE_DONE (gather(l+1) waits for done(l-1), default) or GATE_BEGIN (waits for layer l to begin)."""
        _check("swr_planner_set_gate", lib().swr_planner_set_gate(self._h, int(gate)))

    def set_copy_engine(self, engine: int) -> None:
        """ENGINE_KERNEL (the copy kernel, default) or ENGINE_DMA (the DMA engines)."""
        _check("swr_planner_set_copy_engine", lib().swr_planner_set_copy_engine(self._h, int(engine)))

    def set_gather_lds(self, nbytes: int) -> None:
        """LDS each copy workgroup of the planner's gathers reserves, to leave CUs to the GEMMs (0: none)."""
        _check("swr_planner_set_gather_lds", lib().swr_planner_set_gather_lds(self._h, int(nbytes)))

    def set_timing(self, capacity: int) -> None:
        """Time the copies of the next dispatches in a ring of `capacity` event pairs (0: off)."""
        _check("swr_planner_set_timing", lib().swr_planner_set_timing(self._h, int(capacity)))

    def pause_timing(self, paused: bool) -> None:
        """Records no timing events while paused (the rings keep their contents)."""
        _check("swr_planner_pause_timing", lib().swr_planner_pause_timing(self._h, int(bool(paused))))

    def gather_times(self, cap: int = 1 << 16) -> list[float]:
        """Copy durations (ms) of the timed dispatches still in the ring, oldest first."""
        n = _i32(0)
        buf = (ctypes.c_float * max(cap, 1))()
        _check("swr_planner_gather_times", lib().swr_planner_gather_times(self._h, buf, int(cap), ctypes.byref(n)))
        return list(buf[:n.value])

    def layer_times(self, cap: int = 1 << 16) -> list[float]:
        """Compute spans (ms) of the timed layers still in the ring, oldest first (begin record to done)."""
        n = _i32(0)
        buf = (ctypes.c_float * max(cap, 1))()
        _check("swr_planner_layer_times", lib().swr_planner_layer_times(self._h, buf, int(cap), ctypes.byref(n)))
        return list(buf[:n.value])

    def counters(self) -> tuple[int, int]:
        rb, g = _i64(0), _i64(0)
        _check("swr_planner_counters", lib().swr_planner_counters(self._h, ctypes.byref(rb), ctypes.byref(g)))
        return rb.value, g.value

    def trace(self) -> list[tuple]:
        n = _i32(0)
        _check("swr_planner_trace", lib().swr_planner_trace(self._h, None, 0, ctypes.byref(n)))
        buf = (_i32 * (4 * max(n.value, 1)))()
        _check("swr_planner_trace", lib().swr_planner_trace(self._h, buf, n.value, ctypes.byref(n)))
        return [(TRACE_OPS[buf[4 * i]], TRACE_STREAMS[buf[4 * i + 1]], buf[4 * i + 2], buf[4 * i + 3])
                for i in range(n.value)]

    def close(self) -> None:
        if self._h:
            lib().swr_planner_destroy(self._h)
            self._h = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def version() -> str:
    return lib().swr_version().decode()
