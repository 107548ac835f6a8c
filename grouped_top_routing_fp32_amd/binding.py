"""Thin ctypes binding of libbeam_moe.so (the C ABI in include/beam_moe.h).

Argument marshalling only: torch tensors supply device pointers and the
current HIP stream; every step of the block runs in the library's kernels.
The library is loaded from this package directory and nothing else: when it
is missing or fails to load, every call raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

from .synth import Dims

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libbeam_moe.so")

BEAM_MOE_OK = 0
BEAM_MOE_ERR_INVALID_ARG = -1
BEAM_MOE_ERR_UNSUPPORTED = -2
BEAM_MOE_ERR_WORKSPACE = -3
BEAM_MOE_ERR_HIP = -4
BEAM_MOE_ERR_SCRATCH = -5
SCRATCH_BYTES = 64 << 20       # BEAM_MOE_SCRATCH_BYTES: scratch of beam_moe_forward_noalloc

EXPORTED = ("beam_moe_workspace_bytes", "beam_moe_route_workspace_bytes", "beam_moe_dispatch_workspace_bytes",
            "beam_moe_route", "beam_moe_select", "beam_moe_dispatch",
            "beam_moe_forward", "beam_moe_forward_noalloc", "beam_moe_pack_weights", "beam_moe_forward_packed",
            "beam_moe_forward_fp8", "beam_moe_residual_forward",
            "beam_moe_residual_forward_fp8", "beam_moe_stream_rows", "beam_moe_timing_enable",
            "beam_moe_timing_read", "beam_moe_stage_name", "beam_moe_status_str")

SIZE_MAX = 2 ** 64 - 1


class BeamMoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        self.status = status
        super().__init__(f"{what}: status {status} ({status_text(status)})")


class CDims(ctypes.Structure):
    _fields_ = [("hidden", ctypes.c_int32), ("intermediate", ctypes.c_int32), ("num_experts", ctypes.c_int32),
                ("num_groups", ctypes.c_int32), ("topk_groups", ctypes.c_int32), ("topk", ctypes.c_int32),
                ("routed_scaling", ctypes.c_float)]


_lib: Optional[ctypes.CDLL] = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load the built library (once). Raises if it has not been built."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m grouped_top_routing_fp32_amd.build`")
    lib = ctypes.CDLL(path)
    vp, i32, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
    pd = ctypes.POINTER(CDims)
    for fn in ("beam_moe_workspace_bytes", "beam_moe_route_workspace_bytes", "beam_moe_dispatch_workspace_bytes"):
        getattr(lib, fn).argtypes = [pd, i32]
        getattr(lib, fn).restype = sz
    lib.beam_moe_status_str.argtypes = [ctypes.c_int]
    lib.beam_moe_status_str.restype = ctypes.c_char_p
    lib.beam_moe_route.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.beam_moe_route.restype = ctypes.c_int
    lib.beam_moe_select.argtypes = [pd, i32, vp, vp, vp, vp, vp]
    lib.beam_moe_select.restype = ctypes.c_int
    lib.beam_moe_dispatch.argtypes = [pd, i32, vp, vp, vp, vp, vp, sz, vp]
    lib.beam_moe_dispatch.restype = ctypes.c_int
    lib.beam_moe_forward.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.beam_moe_forward.restype = ctypes.c_int
    lib.beam_moe_pack_weights.argtypes = [pd, vp, vp, vp]
    lib.beam_moe_pack_weights.restype = ctypes.c_int
    lib.beam_moe_forward_packed.argtypes = [pd, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.beam_moe_forward_packed.restype = ctypes.c_int
    lib.beam_moe_forward_noalloc.argtypes = [pd, i32] + [vp] * 13 + [vp]
    lib.beam_moe_forward_noalloc.restype = ctypes.c_int
    lib.beam_moe_forward_fp8.argtypes = [pd, i32] + [vp] * 17 + [sz, vp]
    lib.beam_moe_forward_fp8.restype = ctypes.c_int
    lib.beam_moe_residual_forward.argtypes = [pd, i32, vp, i32, vp, vp, ctypes.c_float, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp, vp, vp, vp, vp, sz, vp]
    lib.beam_moe_residual_forward.restype = ctypes.c_int
    lib.beam_moe_residual_forward_fp8.argtypes = [pd, i32, vp, i32, vp, vp, ctypes.c_float] + [vp] * 16 + [sz, vp]
    lib.beam_moe_residual_forward_fp8.restype = ctypes.c_int
    lib.beam_moe_stream_rows.argtypes = [pd, i32, ctypes.c_int]
    lib.beam_moe_stream_rows.restype = ctypes.c_int
    lib.beam_moe_timing_enable.argtypes = [ctypes.c_int]
    lib.beam_moe_timing_enable.restype = ctypes.c_int
    lib.beam_moe_timing_read.argtypes = [ctypes.POINTER(ctypes.c_float), i32, ctypes.POINTER(i32),
                                         ctypes.POINTER(i32)]
    lib.beam_moe_timing_read.restype = ctypes.c_int
    lib.beam_moe_stage_name.argtypes = [i32]
    lib.beam_moe_stage_name.restype = ctypes.c_char_p
    _lib = lib
    return lib


def status_text(status: int) -> str:
    try:
        return load_library().beam_moe_status_str(status).decode()
    except Exception:  # the message of an error must not itself raise
        return "?"


def _cdims(d: Dims) -> CDims:
    return CDims(d.hidden, d.intermediate, d.num_experts, d.num_groups, d.topk_groups, d.topk,
                 float(d.routed_scaling))


def _ptr(t: Optional[torch.Tensor]):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, what: str) -> None:
    if status != BEAM_MOE_OK:
        raise BeamMoeError(status, what)


def _req(t: torch.Tensor, name: str, dtype: torch.dtype, shape) -> None:
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


# --------------------------------------------------------------------------
# raw entry points (same names as the C ABI)
# --------------------------------------------------------------------------
def _ws_query(fn: str, dims: Dims, T: int) -> int:
    cd = _cdims(dims)
    n = getattr(load_library(), fn)(ctypes.byref(cd), int(T))
    if n == SIZE_MAX:
        raise BeamMoeError(BEAM_MOE_ERR_UNSUPPORTED, fn)
    return int(n)


def beam_moe_workspace_bytes(dims: Dims, T: int) -> int:
    return _ws_query("beam_moe_workspace_bytes", dims, T)


def beam_moe_route_workspace_bytes(dims: Dims, T: int) -> int:
    return _ws_query("beam_moe_route_workspace_bytes", dims, T)


def beam_moe_dispatch_workspace_bytes(dims: Dims, T: int) -> int:
    return _ws_query("beam_moe_dispatch_workspace_bytes", dims, T)


def beam_moe_status_str(status: int) -> str:
    return status_text(status)


def workspace(dims: Dims, T: int, device="cuda", size_fn=None) -> torch.Tensor:
    """A uint8 device buffer of size_fn(dims, T) bytes (default beam_moe_workspace_bytes)."""
    n = (size_fn or beam_moe_workspace_bytes)(dims, T)
    return torch.empty(max(16, n), dtype=torch.uint8, device=device)


def beam_moe_route(dims: Dims, x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor] = None,
                   *, select_bias: Optional[torch.Tensor] = None, want_scores: bool = False,
                   ws: Optional[torch.Tensor] = None, stream=None):
    """Router + group-limited top-k. Returns (ids [T,K] int32, w [T,K] f32, scores [T,E] f32 or None)."""
    T = x.shape[0]
    H, E, K = dims.hidden, dims.num_experts, dims.topk
    _req(x, "x", torch.bfloat16, (T, H))
    _req(w_router, "w_router", torch.float32, (E, H))
    if logit_bias is not None:
        _req(logit_bias, "logit_bias", torch.float32, (E,))
    if select_bias is not None:
        _req(select_bias, "select_bias", torch.float32, (E,))
    dev = x.device
    ids = torch.empty((T, K), dtype=torch.int32, device=dev)
    w = torch.empty((T, K), dtype=torch.float32, device=dev)
    scores = torch.empty((T, E), dtype=torch.float32, device=dev) if want_scores else None
    if ws is None:
        ws = workspace(dims, T, dev, beam_moe_route_workspace_bytes)
    cd = _cdims(dims)
    st = load_library().beam_moe_route(ctypes.byref(cd), T, _ptr(x), _ptr(w_router), _ptr(logit_bias),
                                       _ptr(select_bias), _ptr(ids), _ptr(w), _ptr(scores), _ptr(ws), ws.numel(),
                                       _stream(stream))
    _check(st, "beam_moe_route")
    return ids, w, scores


def beam_moe_select(dims: Dims, scores: torch.Tensor, *, select_bias: Optional[torch.Tensor] = None, stream=None):
    """Selection on supplied post-sigmoid FP32 scores [T,E]. Returns (ids, w)."""
    T = scores.shape[0]
    _req(scores, "scores", torch.float32, (T, dims.num_experts))
    if select_bias is not None:
        _req(select_bias, "select_bias", torch.float32, (dims.num_experts,))
    ids = torch.empty((T, dims.topk), dtype=torch.int32, device=scores.device)
    w = torch.empty((T, dims.topk), dtype=torch.float32, device=scores.device)
    cd = _cdims(dims)
    st = load_library().beam_moe_select(ctypes.byref(cd), T, _ptr(scores), _ptr(select_bias), _ptr(ids), _ptr(w),
                                        _stream(stream))
    _check(st, "beam_moe_select")
    return ids, w


def beam_moe_dispatch(dims: Dims, topk_ids: torch.Tensor, *, ws: Optional[torch.Tensor] = None, stream=None):
    """Counting-sort dispatch. Returns (counts [E], offsets [E+1], sorted_slots [T*K]) int32."""
    T = topk_ids.shape[0]
    _req(topk_ids, "topk_ids", torch.int32, (T, dims.topk))
    dev = topk_ids.device
    E = dims.num_experts
    counts = torch.empty((E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((E + 1,), dtype=torch.int32, device=dev)
    slots = torch.empty((T * dims.topk,), dtype=torch.int32, device=dev)
    if ws is None:
        ws = workspace(dims, T, dev, beam_moe_dispatch_workspace_bytes)
    cd = _cdims(dims)
    st = load_library().beam_moe_dispatch(ctypes.byref(cd), T, _ptr(topk_ids), _ptr(counts), _ptr(offsets),
                                          _ptr(slots), _ptr(ws), ws.numel(), _stream(stream))
    _check(st, "beam_moe_dispatch")
    return counts, offsets, slots


class ForwardBuffers:
    """Caller-owned outputs and workspace of beam_moe_forward for T tokens."""

    def __init__(self, dims: Dims, T: int, device="cuda"):
        E, K, H = dims.num_experts, dims.topk, dims.hidden
        self.T = T
        self.out = torch.empty((T, H), dtype=torch.float32, device=device)
        self.ids = torch.empty((T, K), dtype=torch.int32, device=device)
        self.w = torch.empty((T, K), dtype=torch.float32, device=device)
        self.counts = torch.empty((E,), dtype=torch.int32, device=device)
        self.offsets = torch.empty((E + 1,), dtype=torch.int32, device=device)
        self.slots = torch.empty((T * K,), dtype=torch.int32, device=device)
        self.ws = workspace(dims, T, device)


def _req_router(dims: Dims, w_router, logit_bias, select_bias) -> None:
    E, H = dims.num_experts, dims.hidden
    _req(w_router, "w_router", torch.float32, (E, H))
    for t, name in ((logit_bias, "logit_bias"), (select_bias, "select_bias")):
        if t is not None:
            _req(t, name, torch.float32, (E,))


def _req_bf16_experts(dims: Dims, w_gate, w_up, w_down) -> None:
    E, I, H = dims.num_experts, dims.intermediate, dims.hidden
    _req(w_gate, "w_gate", torch.bfloat16, (E, I, H))
    _req(w_up, "w_up", torch.bfloat16, (E, I, H))
    _req(w_down, "w_down", torch.bfloat16, (E, H, I))


def _req_fp8_experts(dims: Dims, w_gate_fp8, gate_scale, w_up_fp8, up_scale, w_down_fp8, down_scale) -> None:
    E, I, H = dims.num_experts, dims.intermediate, dims.hidden
    _req(w_gate_fp8, "w_gate_fp8", torch.uint8, (E, I, H))
    _req(w_up_fp8, "w_up_fp8", torch.uint8, (E, I, H))
    _req(w_down_fp8, "w_down_fp8", torch.uint8, (E, H, I))
    _req(gate_scale, "gate_scale", torch.float32, (E, I))
    _req(up_scale, "up_scale", torch.float32, (E, I))
    _req(down_scale, "down_scale", torch.float32, (E, H))


def _buffers(dims: Dims, T: int, device, bufs: Optional[ForwardBuffers]) -> ForwardBuffers:
    if bufs is None:
        return ForwardBuffers(dims, T, device)
    if bufs.T != T:
        raise ValueError("buffers were sized for another T")
    return bufs


def _outputs(bufs: ForwardBuffers, out: torch.Tensor):
    """Pointer arguments from `out` through the workspace, as every forward entry point takes them."""
    return (_ptr(out), _ptr(bufs.ids), _ptr(bufs.w), _ptr(bufs.counts), _ptr(bufs.offsets), _ptr(bufs.slots),
            _ptr(bufs.ws), bufs.ws.numel())


def beam_moe_forward(dims: Dims, x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor],
                     w_gate: torch.Tensor, w_up: torch.Tensor, w_down: torch.Tensor, *,
                     select_bias: Optional[torch.Tensor] = None, bufs: Optional[ForwardBuffers] = None,
                     stream=None) -> ForwardBuffers:
    """The whole block. Returns the ForwardBuffers holding out and the routing by-products."""
    T = x.shape[0]
    _req(x, "x", torch.bfloat16, (T, dims.hidden))
    _req_router(dims, w_router, logit_bias, select_bias)
    _req_bf16_experts(dims, w_gate, w_up, w_down)
    bufs = _buffers(dims, T, x.device, bufs)
    cd = _cdims(dims)
    st = load_library().beam_moe_forward(
        ctypes.byref(cd), T, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), *_outputs(bufs, bufs.out), _stream(stream))
    _check(st, "beam_moe_forward")
    return bufs


def beam_moe_pack_weights(dims: Dims, w_down: torch.Tensor, out: Optional[torch.Tensor] = None,
                          stream=None) -> torch.Tensor:
    """W_down [E, H, I] bf16 -> fp16 (the form beam_moe_forward_packed takes)."""
    E, I, H = dims.num_experts, dims.intermediate, dims.hidden
    _req(w_down, "w_down", torch.bfloat16, (E, H, I))
    if out is None:
        out = torch.empty((E, H, I), dtype=torch.float16, device=w_down.device)
    _req(out, "w_down_packed", torch.float16, (E, H, I))
    cd = _cdims(dims)
    _check(load_library().beam_moe_pack_weights(ctypes.byref(cd), _ptr(w_down), _ptr(out), _stream(stream)),
           "beam_moe_pack_weights")
    return out


def beam_moe_forward_packed(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                            logit_bias: Optional[torch.Tensor], w_gate: torch.Tensor, w_up: torch.Tensor,
                            w_down_packed: torch.Tensor, *, select_bias: Optional[torch.Tensor] = None,
                            bufs: Optional[ForwardBuffers] = None, stream=None) -> ForwardBuffers:
    """beam_moe_forward with W_down from beam_moe_pack_weights (fp16)."""
    T = x.shape[0]
    E, I, H = dims.num_experts, dims.intermediate, dims.hidden
    _req(x, "x", torch.bfloat16, (T, H))
    _req_router(dims, w_router, logit_bias, select_bias)
    _req(w_gate, "w_gate", torch.bfloat16, (E, I, H))
    _req(w_up, "w_up", torch.bfloat16, (E, I, H))
    _req(w_down_packed, "w_down_packed", torch.float16, (E, H, I))
    bufs = _buffers(dims, T, x.device, bufs)
    cd = _cdims(dims)
    st = load_library().beam_moe_forward_packed(
        ctypes.byref(cd), T, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down_packed), *_outputs(bufs, bufs.out), _stream(stream))
    _check(st, "beam_moe_forward_packed")
    return bufs


def beam_moe_forward_noalloc(dims: Dims, x: torch.Tensor, w_router: torch.Tensor,
                             logit_bias: Optional[torch.Tensor], w_gate: torch.Tensor, w_up: torch.Tensor,
                             w_down: torch.Tensor, *, select_bias: Optional[torch.Tensor] = None,
                             bufs: Optional[ForwardBuffers] = None, stream=None) -> ForwardBuffers:
    """beam_moe_forward on the library's built-in scratch (no workspace); bufs.ws is not used."""
    T = x.shape[0]
    _req(x, "x", torch.bfloat16, (T, dims.hidden))
    _req_router(dims, w_router, logit_bias, select_bias)
    _req_bf16_experts(dims, w_gate, w_up, w_down)
    bufs = _buffers(dims, T, x.device, bufs)
    cd = _cdims(dims)
    st = load_library().beam_moe_forward_noalloc(
        ctypes.byref(cd), T, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), *_outputs(bufs, bufs.out)[:6], _stream(stream))
    _check(st, "beam_moe_forward_noalloc")
    return bufs


def beam_moe_forward_fp8(dims: Dims, x: torch.Tensor, w_router: torch.Tensor, logit_bias: Optional[torch.Tensor],
                         w_gate_fp8: torch.Tensor, gate_scale: torch.Tensor, w_up_fp8: torch.Tensor,
                         up_scale: torch.Tensor, w_down_fp8: torch.Tensor, down_scale: torch.Tensor, *,
                         select_bias: Optional[torch.Tensor] = None, bufs: Optional[ForwardBuffers] = None,
                         stream=None) -> ForwardBuffers:
    """The whole block with E4M3 expert weights (uint8 codes) and fp32 per-row scales."""
    T = x.shape[0]
    _req(x, "x", torch.bfloat16, (T, dims.hidden))
    _req_router(dims, w_router, logit_bias, select_bias)
    _req_fp8_experts(dims, w_gate_fp8, gate_scale, w_up_fp8, up_scale, w_down_fp8, down_scale)
    bufs = _buffers(dims, T, x.device, bufs)
    cd = _cdims(dims)
    st = load_library().beam_moe_forward_fp8(
        ctypes.byref(cd), T, _ptr(x), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate_fp8),
        _ptr(gate_scale), _ptr(w_up_fp8), _ptr(up_scale), _ptr(w_down_fp8), _ptr(down_scale),
        *_outputs(bufs, bufs.out), _stream(stream))
    _check(st, "beam_moe_forward_fp8")
    return bufs


def _residual_prelude(dims: Dims, stream_in, norm_in_weight, norm_out_weight, stream_out, bufs):
    T = stream_in.shape[0]
    H = dims.hidden
    _req(stream_in, "stream_in", torch.float32, (T, H))
    for t, name in ((norm_in_weight, "norm_in_weight"), (norm_out_weight, "norm_out_weight")):
        if t is not None:
            _req(t, name, torch.float32, (H,))
    bufs = _buffers(dims, T, stream_in.device, bufs)
    if stream_out is not None:
        _req(stream_out, "stream_out", torch.float32, (T, H))
    return T, bufs, (stream_out if stream_out is not None else bufs.out)


def beam_moe_residual_forward(dims: Dims, stream_in: torch.Tensor, step: int, w_router: torch.Tensor,
                              logit_bias: Optional[torch.Tensor], w_gate: torch.Tensor, w_up: torch.Tensor,
                              w_down: torch.Tensor, *, select_bias: Optional[torch.Tensor] = None,
                              norm_in_weight: Optional[torch.Tensor] = None,
                              norm_out_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                              stream_out: Optional[torch.Tensor] = None, bufs: Optional[ForwardBuffers] = None,
                              stream=None) -> ForwardBuffers:
    """The block as a residual sublayer at `step`: the new stream goes to stream_out if given (it may be
    stream_in itself), else to bufs.out; the routing by-products to bufs."""
    T, bufs, out = _residual_prelude(dims, stream_in, norm_in_weight, norm_out_weight, stream_out, bufs)
    _req_router(dims, w_router, logit_bias, select_bias)
    _req_bf16_experts(dims, w_gate, w_up, w_down)
    cd = _cdims(dims)
    st = load_library().beam_moe_residual_forward(
        ctypes.byref(cd), T, _ptr(stream_in), int(step), _ptr(norm_in_weight), _ptr(norm_out_weight),
        float(norm_eps), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate), _ptr(w_up),
        _ptr(w_down), *_outputs(bufs, out), _stream(stream))
    _check(st, "beam_moe_residual_forward")
    return bufs


def beam_moe_residual_forward_fp8(dims: Dims, stream_in: torch.Tensor, step: int, w_router: torch.Tensor,
                                  logit_bias: Optional[torch.Tensor], w_gate_fp8: torch.Tensor,
                                  gate_scale: torch.Tensor, w_up_fp8: torch.Tensor, up_scale: torch.Tensor,
                                  w_down_fp8: torch.Tensor, down_scale: torch.Tensor, *,
                                  select_bias: Optional[torch.Tensor] = None,
                                  norm_in_weight: Optional[torch.Tensor] = None,
                                  norm_out_weight: Optional[torch.Tensor] = None, norm_eps: float = 1e-6,
                                  stream_out: Optional[torch.Tensor] = None, bufs: Optional[ForwardBuffers] = None,
                                  stream=None) -> ForwardBuffers:
    """beam_moe_residual_forward with E4M3 expert weights and fp32 per-row scales."""
    T, bufs, out = _residual_prelude(dims, stream_in, norm_in_weight, norm_out_weight, stream_out, bufs)
    _req_router(dims, w_router, logit_bias, select_bias)
    _req_fp8_experts(dims, w_gate_fp8, gate_scale, w_up_fp8, up_scale, w_down_fp8, down_scale)
    cd = _cdims(dims)
    st = load_library().beam_moe_residual_forward_fp8(
        ctypes.byref(cd), T, _ptr(stream_in), int(step), _ptr(norm_in_weight), _ptr(norm_out_weight),
        float(norm_eps), _ptr(w_router), _ptr(logit_bias), _ptr(select_bias), _ptr(w_gate_fp8), _ptr(gate_scale),
        _ptr(w_up_fp8), _ptr(up_scale), _ptr(w_down_fp8), _ptr(down_scale), *_outputs(bufs, out), _stream(stream))
    _check(st, "beam_moe_residual_forward_fp8")
    return bufs


# --------------------------------------------------------------------------
# stage timing diagnostics
# --------------------------------------------------------------------------
def beam_moe_stream_rows(dims: Dims, T: int, fp8: bool = False) -> int:
    """Rows per stream-kernel tile the forward entry points use for T tokens, or 0 for the grouped GEMMs."""
    cd = _cdims(dims)
    r = load_library().beam_moe_stream_rows(ctypes.byref(cd), int(T), int(bool(fp8)))
    if r < 0:
        raise BeamMoeError(r, "beam_moe_stream_rows")
    return r


def beam_moe_timing_enable(enable: bool = True) -> None:
    _check(load_library().beam_moe_timing_enable(int(bool(enable))), "beam_moe_timing_enable")


def beam_moe_stage_name(stage: int) -> Optional[str]:
    r = load_library().beam_moe_stage_name(stage)
    return None if r is None else r.decode()


def beam_moe_timing_read() -> tuple[dict, int]:
    """({stage name: summed ms}, calls) since the previous read; waits for the last recorded call."""
    buf = (ctypes.c_float * 16)()
    ns, calls = ctypes.c_int32(0), ctypes.c_int32(0)
    _check(load_library().beam_moe_timing_read(buf, 16, ctypes.byref(ns), ctypes.byref(calls)),
           "beam_moe_timing_read")
    return {beam_moe_stage_name(i): float(buf[i]) for i in range(ns.value)}, calls.value
