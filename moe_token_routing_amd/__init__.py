"""MoE routing-and-combine hot path on MI355X (gfx950).

A thin Python binding over the C ABI of libmoe_routing.so (declared in
include/moe_routing.h). Every step runs in the library's HIP kernels; this
module only checks tensors, allocates outputs when the caller did not pass
them, and forwards raw device pointers and the current HIP stream. PyTorch
supplies device memory and streams.

The library must be built first (``python -m moe_token_routing_amd.build`` or
``__graft_entry__.build()``); importing the binding without it raises.
"""
from __future__ import annotations

import ctypes
import os
from typing import Optional

import torch

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libmoe_routing.so")

MOE_DTYPE_F32 = 0
MOE_DTYPE_BF16 = 1
MAX_EXPERTS = 4096
MAX_TOPK = 32
MAX_HIDDEN = 16384

_lib = None

_c_int, _c_float, _c_size, _vp = ctypes.c_int, ctypes.c_float, ctypes.c_size_t, ctypes.c_void_p

_SIGNATURES = {
    "moe_status_string": (ctypes.c_char_p, [_c_int]),
    "moe_route_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_route": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_float, _c_int, _c_int, _c_int, _c_int,
                           _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_dispatch_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "moe_dispatch": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_dispatch_noalloc": (_c_int, [_vp, _c_int, _c_int, _c_int, _vp, _vp, _vp, _vp, _vp]),
    "moe_route_dispatch_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int, _c_int, _c_int, _c_int]),
    "moe_route_dispatch": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_float, _c_int, _c_int, _c_int, _c_int,
                                    _vp, _vp, _vp, _vp, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_route_dispatch_quant": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_float, _c_int, _c_int, _c_int, _c_int,
                                          _vp, _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _c_int, _vp, _c_float, _c_float, _vp, _vp, _vp, _vp, _c_size, _vp]),
    "moe_norm_quant_nvfp4": (_c_int, [_vp, _vp, _c_float, _c_float, _vp, _c_int, _c_int, _vp, _vp, _vp]),
    "moe_norm_quant_nvfp4_rank_block": (_c_int, [_vp, _c_int, _vp, _c_float, _c_float, _vp, _c_int, _c_int,
                                                 _vp, _vp, _vp]),
    "moe_combine": (_c_int, [_vp, _c_int, _vp, _vp, _vp, _c_float, _c_float, _c_int, _c_int, _c_int,
                             _vp, _vp]),
    "moe_expert_fc1_workspace_bytes": (_c_size, [_c_int, _c_int, _c_int]),
    "moe_expert_fc1_nvfp4": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                      _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]),
    "moe_expert_fc1_swiglu_nvfp4": (_c_int, [_vp, _vp, _vp, _vp, _vp, _c_int, _c_int, _vp, _vp, _vp, _vp,
                                             _c_int, _c_int, _c_int, _vp, _vp, _vp, _c_size, _vp]),
}


class MoeError(RuntimeError):
    """A call returned a nonzero status."""

    def __init__(self, fn: str, status: int):
        self.status = status
        super().__init__("%s failed: %s (status %d)" % (fn, status_string(status), status))


def lib() -> ctypes.CDLL:
    """The loaded library (loaded on first use; raises if it was not built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError("libmoe_routing.so is not built; run `python -m moe_token_routing_amd.build`")
        handle = ctypes.CDLL(LIB_PATH)
        for name, (res, args) in _SIGNATURES.items():
            fn = getattr(handle, name)
            fn.restype = res
            fn.argtypes = args
        _lib = handle
    return _lib


def status_string(status: int) -> str:
    return lib().moe_status_string(status).decode()


def _check(fn: str, status: int):
    if status != 0:
        raise MoeError(fn, status)


# The checks and conversions below run on every call, so they take the
# cheapest route to the same facts (a decode-sized call's own host work is a
# few microseconds; these helpers had cost about twice that).

def _ptr(t: Optional[torch.Tensor]):
    # a plain int: ctypes converts it for the c_void_p parameter
    return None if t is None else t.data_ptr()


try:
    _raw_stream = torch._C._cuda_getCurrentRawStream
except AttributeError:   # older torch: the public query (slower)
    def _raw_stream(index):
        return torch.cuda.current_stream(index).cuda_stream


def _stream(device: torch.device):
    """The device's current HIP stream, as a raw handle."""
    return _raw_stream(device.index if device.index is not None else torch.cuda.current_device())


def _need(t: torch.Tensor, name: str, dtypes, shape=None, device=None):
    try:
        if (t.is_cuda and t.dtype in dtypes and t.is_contiguous() and (shape is None or t.shape == tuple(shape))
                and (device is None or t.device == device)):
            return
    except AttributeError:
        pass
    _need_failed(t, name, dtypes, shape, device)


def _need_failed(t, name, dtypes, shape, device):
    if not isinstance(t, torch.Tensor):
        raise TypeError("%s must be a tensor" % name)
    if t.device.type != "cuda":
        raise ValueError("%s must be a GPU tensor" % name)
    if device is not None and t.device != device:
        raise ValueError("%s is on %s, expected %s" % (name, t.device, device))
    if t.dtype not in dtypes:
        raise TypeError("%s has dtype %s, expected one of %s" % (name, t.dtype, dtypes))
    if not t.is_contiguous():
        raise ValueError("%s must be contiguous" % name)
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError("%s has shape %s, expected %s" % (name, tuple(t.shape), tuple(shape)))
    raise AssertionError("%s failed a check that names no reason" % name)


_BF16 = (torch.bfloat16, torch.int16, torch.uint16)


def route_workspace_bytes(T: int, H: int, E: int, k: int, hidden_dtype: int, logits_in: bool = False) -> int:
    return int(lib().moe_route_workspace_bytes(T, H, E, k, hidden_dtype, int(bool(logits_in))))


def _route_io(hidden, W, bias, token_mask, k, logits, topk_ids, topk_w):
    """Checks and allocates moe_route's arguments; returns (T, H, E, dtype,
    logits, topk_ids, topk_w)."""
    dev = bias.device
    E = bias.shape[0]
    _need(bias, "bias", (torch.float32,), (E,))
    T = token_mask.shape[0]
    _need(token_mask, "token_mask", (torch.uint8, torch.bool), (T,), dev)
    if hidden is None:
        if logits is None:
            raise ValueError("logits-in mode needs logits")
        _need(logits, "logits", (torch.float32,), (T, E), dev)
        H = 16
        dtype = MOE_DTYPE_BF16
    else:
        _need(hidden, "hidden", (torch.float32,) + _BF16, None, dev)
        if hidden.dim() != 2 or hidden.shape[0] != T:
            raise ValueError("hidden must be [T,H] with T = len(token_mask)")
        H = hidden.shape[1]
        dtype = MOE_DTYPE_F32 if hidden.dtype == torch.float32 else MOE_DTYPE_BF16
        _need(W, "W", (torch.float32,), (E, H), dev)
        if logits is None:
            logits = torch.empty((T, E), dtype=torch.float32, device=dev)
        _need(logits, "logits", (torch.float32,), (T, E), dev)
    if topk_ids is None:
        topk_ids = torch.empty((T, k), dtype=torch.int32, device=dev)
    if topk_w is None:
        topk_w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _need(topk_ids, "topk_ids", (torch.int32,), (T, k), dev)
    _need(topk_w, "topk_w", (torch.float32,), (T, k), dev)
    return T, H, E, dtype, logits, topk_ids, topk_w


def _dispatch_io(dev, T, k, E, counts, offsets, perm, dest):
    """Checks and allocates moe_dispatch's outputs."""
    n = T * k
    counts = torch.empty(E, dtype=torch.int32, device=dev) if counts is None else counts
    offsets = torch.empty(E + 1, dtype=torch.int32, device=dev) if offsets is None else offsets
    perm = torch.empty(n, dtype=torch.int32, device=dev) if perm is None else perm
    dest = torch.empty(n, dtype=torch.int32, device=dev) if dest is None else dest
    _need(counts, "counts", (torch.int32,), (E,), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    _need(perm, "perm", (torch.int32,), (n,), dev)
    _need(dest, "dest", (torch.int32,), (n,), dev)
    return counts, offsets, perm, dest


def _workspace(workspace, ws_bytes, dev):
    if workspace is None and ws_bytes > 0:
        workspace = torch.empty(ws_bytes, dtype=torch.uint8, device=dev)
    ws_len = 0 if workspace is None else workspace.numel() * workspace.element_size()
    return workspace, ws_len


def route(hidden: Optional[torch.Tensor], W: Optional[torch.Tensor], bias: torch.Tensor,
          token_mask: torch.Tensor, k: int, scale: float = 1.0, *, logits: Optional[torch.Tensor] = None,
          topk_ids: Optional[torch.Tensor] = None, topk_w: Optional[torch.Tensor] = None,
          workspace: Optional[torch.Tensor] = None):
    """moe_route. hidden: [T,H] bf16 or fp32 (None: logits-in mode, `logits`
    [T,E] fp32 is then an input). Returns (logits, topk_ids int32, topk_w fp32)."""
    dev = bias.device
    T, H, E, dtype, logits, topk_ids, topk_w = _route_io(hidden, W, bias, token_mask, k, logits, topk_ids, topk_w)
    workspace, ws_len = _workspace(workspace, route_workspace_bytes(T, H, E, k, dtype, hidden is None), dev)
    _check("moe_route", lib().moe_route(
        _ptr(hidden), dtype, _ptr(W), _ptr(bias), _ptr(token_mask), float(scale), T, H, E, k,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(workspace), ws_len, _stream(dev)))
    return logits, topk_ids, topk_w


def dispatch_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_dispatch_workspace_bytes(T, k, E))


def dispatch(topk_ids: torch.Tensor, E: int, *, counts=None, offsets=None, perm=None, dest=None,
             workspace: Optional[torch.Tensor] = None):
    """moe_dispatch. Returns (counts [E], offsets [E+1], perm [T*k], dest [T*k]), int32."""
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", (torch.int32,), None, dev)
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T,k]")
    T, k = topk_ids.shape
    counts, offsets, perm, dest = _dispatch_io(dev, T, k, E, counts, offsets, perm, dest)
    workspace, ws_len = _workspace(workspace, dispatch_workspace_bytes(T, k, E), dev)
    _check("moe_dispatch", lib().moe_dispatch(
        _ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(dest),
        _ptr(workspace), ws_len, _stream(dev)))
    return counts, offsets, perm, dest


def dispatch_noalloc(topk_ids: torch.Tensor, E: int, *, counts=None, offsets=None, perm=None, dest=None):
    """moe_dispatch_noalloc: moe_dispatch with the library's static device
    scratch instead of a workspace (outputs are allocated here when not
    given, as in dispatch()). Returns (counts, offsets, perm, dest)."""
    dev = topk_ids.device
    _need(topk_ids, "topk_ids", (torch.int32,), None, dev)
    if topk_ids.dim() != 2:
        raise ValueError("topk_ids must be [T,k]")
    T, k = topk_ids.shape
    counts, offsets, perm, dest = _dispatch_io(dev, T, k, E, counts, offsets, perm, dest)
    _check("moe_dispatch_noalloc", lib().moe_dispatch_noalloc(
        _ptr(topk_ids), T, k, E, _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(dest), _stream(dev)))
    return counts, offsets, perm, dest


def route_dispatch_workspace_bytes(T: int, H: int, E: int, k: int, hidden_dtype: int,
                                   logits_in: bool = False) -> int:
    return int(lib().moe_route_dispatch_workspace_bytes(T, H, E, k, hidden_dtype, int(bool(logits_in))))


def route_dispatch(hidden: Optional[torch.Tensor], W: Optional[torch.Tensor], bias: torch.Tensor,
                   token_mask: torch.Tensor, k: int, scale: float = 1.0, *, logits=None, topk_ids=None,
                   topk_w=None, counts=None, offsets=None, perm=None, dest=None,
                   workspace: Optional[torch.Tensor] = None):
    """moe_route_dispatch: route() then dispatch() of its ids in one call.
    Returns (logits, topk_ids, topk_w, counts, offsets, perm, dest)."""
    dev = bias.device
    T, H, E, dtype, logits, topk_ids, topk_w = _route_io(hidden, W, bias, token_mask, k, logits, topk_ids, topk_w)
    counts, offsets, perm, dest = _dispatch_io(dev, T, k, E, counts, offsets, perm, dest)
    workspace, ws_len = _workspace(workspace, route_dispatch_workspace_bytes(T, H, E, k, dtype, hidden is None),
                                   dev)
    _check("moe_route_dispatch", lib().moe_route_dispatch(
        _ptr(hidden), dtype, _ptr(W), _ptr(bias), _ptr(token_mask), float(scale), T, H, E, k,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(dest),
        _ptr(workspace), ws_len, _stream(dev)))
    return logits, topk_ids, topk_w, counts, offsets, perm, dest


def route_dispatch_quant(hidden: Optional[torch.Tensor], W: Optional[torch.Tensor], bias: torch.Tensor,
                         token_mask: torch.Tensor, k: int, x: torch.Tensor, norm_w: torch.Tensor,
                         gain_center: float, eps: float, global_scale: torch.Tensor, scale: float = 1.0, *,
                         logits=None, topk_ids=None, topk_w=None, counts=None, offsets=None, perm=None, dest=None,
                         packed=None, scales=None, workspace: Optional[torch.Tensor] = None):
    """moe_route_dispatch_quant: route_dispatch() and norm_quant_nvfp4() of x
    in one call. x [T,Hq] bf16 with hidden's T and a width of its own.
    Returns (logits, topk_ids, topk_w, counts, offsets, perm, dest, packed,
    scales)."""
    dev = bias.device
    T, H, E, dtype, logits, topk_ids, topk_w = _route_io(hidden, W, bias, token_mask, k, logits, topk_ids, topk_w)
    counts, offsets, perm, dest = _dispatch_io(dev, T, k, E, counts, offsets, perm, dest)
    _need(x, "x", _BF16, None, dev)
    if x.dim() != 2 or x.shape[0] != T:
        raise ValueError("x must be [T,Hq] with hidden's T")
    Hx = x.shape[1]
    _need(norm_w, "norm_w", (torch.float32,), (Hx,), dev)
    _need(global_scale, "global_scale", (torch.float32,), (1,), dev)
    packed = torch.empty((T, Hx // 2), dtype=torch.uint8, device=dev) if packed is None else packed
    scales = torch.empty((T, Hx // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    _need(packed, "packed", (torch.uint8,), (T, Hx // 2), dev)
    _need(scales, "scales", (torch.uint8,), (T, Hx // 16), dev)
    workspace, ws_len = _workspace(workspace, route_dispatch_workspace_bytes(T, H, E, k, dtype, hidden is None),
                                   dev)
    _check("moe_route_dispatch_quant", lib().moe_route_dispatch_quant(
        _ptr(hidden), dtype, _ptr(W), _ptr(bias), _ptr(token_mask), float(scale), T, H, E, k,
        _ptr(logits), _ptr(topk_ids), _ptr(topk_w), _ptr(counts), _ptr(offsets), _ptr(perm), _ptr(dest),
        _ptr(x), Hx, _ptr(norm_w), float(gain_center), float(eps), _ptr(global_scale), _ptr(packed), _ptr(scales),
        _ptr(workspace), ws_len, _stream(dev)))
    return logits, topk_ids, topk_w, counts, offsets, perm, dest, packed, scales


def norm_quant_nvfp4(x: torch.Tensor, norm_w: torch.Tensor, gain_center: float, eps: float,
                     global_scale: torch.Tensor, *, packed=None, scales=None):
    """moe_norm_quant_nvfp4. x [T,H] bf16; global_scale a 1-element fp32 GPU
    tensor. Returns (packed [T,H/2] uint8, scales [T,H/16] uint8 E4M3)."""
    dev = x.device
    _need(x, "x", _BF16, None, dev)
    if x.dim() != 2:
        raise ValueError("x must be [T,H]")
    T, H = x.shape
    packed, scales = _norm_quant_outputs(norm_w, global_scale, T, H, packed, scales, dev)
    _check("moe_norm_quant_nvfp4", lib().moe_norm_quant_nvfp4(
        _ptr(x), _ptr(norm_w), float(gain_center), float(eps), _ptr(global_scale), T, H,
        _ptr(packed), _ptr(scales), _stream(dev)))
    return packed, scales


def norm_quant_nvfp4_rank_block(x: torch.Tensor, num_tokens: int, norm_w: torch.Tensor, gain_center: float,
                                eps: float, global_scale: torch.Tensor, *, packed=None, scales=None):
    """moe_norm_quant_nvfp4_rank_block. x is [tp * T, H / tp] bf16 (tp blocks
    of column shards stacked along dim 0; tp = 1 is the contiguous [T,H]);
    H is norm_w's length. Returns (packed [T,H/2], scales [T,H/16])."""
    dev = x.device
    _need(x, "x", _BF16, None, dev)
    if x.dim() != 2:
        raise ValueError("x must be [tp*T, H/tp]")
    T = int(num_tokens)
    H = norm_w.shape[0] if norm_w.dim() == 1 else -1
    shard = x.shape[1]
    if T < 0 or H <= 0 or x.shape[0] * shard != T * H:
        raise ValueError("x holds %d x %d values, not num_tokens * H = %d * %d" % (x.shape[0], shard, T, H))
    packed, scales = _norm_quant_outputs(norm_w, global_scale, T, H, packed, scales, dev)
    _check("moe_norm_quant_nvfp4_rank_block", lib().moe_norm_quant_nvfp4_rank_block(
        _ptr(x), shard, _ptr(norm_w), float(gain_center), float(eps), _ptr(global_scale), T, H,
        _ptr(packed), _ptr(scales), _stream(dev)))
    return packed, scales


def _norm_quant_outputs(norm_w, global_scale, T, H, packed, scales, dev):
    _need(norm_w, "norm_w", (torch.float32,), (H,), dev)
    _need(global_scale, "global_scale", (torch.float32,), None, dev)
    if global_scale.numel() != 1:
        raise ValueError("global_scale must hold one value")
    packed = torch.empty((T, H // 2), dtype=torch.uint8, device=dev) if packed is None else packed
    scales = torch.empty((T, H // 16), dtype=torch.uint8, device=dev) if scales is None else scales
    _need(packed, "packed", (torch.uint8,), (T, H // 2), dev)
    _need(scales, "scales", (torch.uint8,), (T, H // 16), dev)
    return packed, scales


def combine(expert_out: torch.Tensor, slots: torch.Tensor, topk_w: torch.Tensor, norm_w: torch.Tensor,
            gain_center: float, eps: float, *, out=None, rows: Optional[int] = None):
    """moe_combine. expert_out [R,H] bf16; slots [T,k] int32; topk_w [T,k]
    fp32. `rows` overrides R (the number of rows a slot may address; default
    expert_out.shape[0]). Returns out [T,H] bf16."""
    dev = slots.device
    _need(expert_out, "expert_out", _BF16, None, dev)
    if expert_out.dim() != 2:
        raise ValueError("expert_out must be [R,H]")
    R, H = expert_out.shape
    if rows is not None:
        if rows < 0 or rows > R:
            raise ValueError("rows must be within [0, expert_out.shape[0]]")
        R = rows
    _need(slots, "slots", (torch.int32,), None, dev)
    if slots.dim() != 2:
        raise ValueError("slots must be [T,k]")
    T, k = slots.shape
    _need(topk_w, "topk_w", (torch.float32,), (T, k), dev)
    _need(norm_w, "norm_w", (torch.float32,), (H,), dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev) if out is None else out
    _need(out, "out", _BF16, (T, H), dev)
    _check("moe_combine", lib().moe_combine(
        _ptr(expert_out), R, _ptr(slots), _ptr(topk_w), _ptr(norm_w), float(gain_center), float(eps),
        T, H, k, _ptr(out), _stream(dev)))
    return out


def expert_fc1_workspace_bytes(T: int, k: int, E: int) -> int:
    return int(lib().moe_expert_fc1_workspace_bytes(T, k, E))


def expert_fc1_nvfp4(x_packed: torch.Tensor, x_scales: torch.Tensor, x_gs: torch.Tensor,
                     perm: torch.Tensor, offsets: torch.Tensor, k: int,
                     w_packed: torch.Tensor, w_scales: torch.Tensor, w_gs: torch.Tensor,
                     y_gs: torch.Tensor, *, y_packed=None, y_scales=None, workspace=None):
    """moe_expert_fc1_nvfp4. x_packed [T,K/2] / x_scales [T,K/16] uint8 (the
    NVFP4 input), perm [T*k] / offsets [E+1] int32 (moe_dispatch's grouping),
    w_packed [E,N,K/2] / w_scales [E,N,K/16] uint8, w_gs [E] fp32, x_gs and
    y_gs one-element fp32 GPU tensors. Returns (y_packed [T*k,N/2],
    y_scales [T*k,N/16]) uint8 in grouped order."""
    return _expert_fc1("moe_expert_fc1_nvfp4", 1, x_packed, x_scales, x_gs, perm, offsets, k, w_packed,
                       w_scales, w_gs, y_gs, y_packed, y_scales, workspace)


def expert_fc1_swiglu_nvfp4(x_packed: torch.Tensor, x_scales: torch.Tensor, x_gs: torch.Tensor,
                            perm: torch.Tensor, offsets: torch.Tensor, k: int,
                            w_packed: torch.Tensor, w_scales: torch.Tensor, w_gs: torch.Tensor,
                            y_gs: torch.Tensor, *, y_packed=None, y_scales=None, workspace=None):
    """moe_expert_fc1_swiglu_nvfp4. As expert_fc1_nvfp4 with w_packed
    [E,2N,K/2] / w_scales [E,2N,K/16] (gate rows, then up rows). Returns
    (y_packed [T*k,N/2], y_scales [T*k,N/16]) uint8 in grouped order."""
    return _expert_fc1("moe_expert_fc1_swiglu_nvfp4", 2, x_packed, x_scales, x_gs, perm, offsets, k, w_packed,
                       w_scales, w_gs, y_gs, y_packed, y_scales, workspace)


def _expert_fc1(fn, rows_per_col, x_packed, x_scales, x_gs, perm, offsets, k, w_packed, w_scales, w_gs, y_gs,
                y_packed, y_scales, workspace):
    dev = x_packed.device
    if x_packed.dim() != 2 or w_packed.dim() != 3:
        raise ValueError("x_packed must be [T,K/2] and w_packed [E,rows,K/2]")
    T, K = x_packed.shape[0], x_packed.shape[1] * 2
    E, rows = w_packed.shape[0], w_packed.shape[1]
    if rows % rows_per_col:
        raise ValueError("w_packed must hold gate and up rows (an even count)")
    N = rows // rows_per_col
    _need(x_packed, "x_packed", (torch.uint8,), (T, K // 2), dev)
    _need(x_scales, "x_scales", (torch.uint8,), (T, K // 16), dev)
    _need(w_packed, "w_packed", (torch.uint8,), (E, rows, K // 2), dev)
    _need(w_scales, "w_scales", (torch.uint8,), (E, rows, K // 16), dev)
    _need(w_gs, "w_gs", (torch.float32,), (E,), dev)
    _need(perm, "perm", (torch.int32,), (T * k,), dev)
    _need(offsets, "offsets", (torch.int32,), (E + 1,), dev)
    for name, g in (("x_gs", x_gs), ("y_gs", y_gs)):
        _need(g, name, (torch.float32,), None, dev)
        if g.numel() != 1:
            raise ValueError(name + " must hold one value")
    P = T * k
    y_packed = torch.empty((P, N // 2), dtype=torch.uint8, device=dev) if y_packed is None else y_packed
    y_scales = torch.empty((P, N // 16), dtype=torch.uint8, device=dev) if y_scales is None else y_scales
    _need(y_packed, "y_packed", (torch.uint8,), (P, N // 2), dev)
    _need(y_scales, "y_scales", (torch.uint8,), (P, N // 16), dev)
    need = expert_fc1_workspace_bytes(T, int(k), E)
    if workspace is None:
        workspace = torch.empty(max(need, 1), dtype=torch.uint8, device=dev)
    _check(fn, getattr(lib(), fn)(
        _ptr(x_packed), _ptr(x_scales), _ptr(x_gs), _ptr(perm), _ptr(offsets), T, int(k),
        _ptr(w_packed), _ptr(w_scales), _ptr(w_gs), _ptr(y_gs), K, N, E,
        _ptr(y_packed), _ptr(y_scales), _ptr(workspace), workspace.numel(), _stream(dev)))
    return y_packed, y_scales
