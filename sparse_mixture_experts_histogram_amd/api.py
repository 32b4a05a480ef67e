"""Torch-facing wrappers with the names of the C entry points.

Tensors provide device memory and the stream; each wrapper checks shapes and
dtypes, allocates outputs and workspace with ``torch.empty`` and calls the
library.  No arithmetic of the layer happens here.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass
from typing import Optional, Sequence, Tuple

import torch

from . import _lib
from ._lib import MoeDesc, MoeError

_DT = {torch.float32: _lib.MOE_F32, torch.bfloat16: _lib.MOE_BF16}
_PATHS = {"auto": _lib.PATH_AUTO, "prefill": _lib.PATH_PREFILL, "decode": _lib.PATH_DECODE}
_SCORING = {"softmax": _lib.SCORING_SOFTMAX, "sigmoid": _lib.SCORING_SIGMOID}


@dataclass(frozen=True)
class Routing:
    """Router options: ``scoring`` "softmax" (default) or "sigmoid" (the bias
    then steers selection only); ``renormalize`` False keeps the raw kept
    scores; ``capacity_factor`` > 0 caps each expert at
    ceil(T*k/E*capacity_factor) pairs (0: dropless)."""
    scoring: str = "softmax"
    renormalize: bool = True
    capacity_factor: float = 0.0


def make_desc(T: int, d: int, E: int, k: int, ffn: int, n_shared: int = 0, ffn_shared: int = 0,
              dtype=torch.bfloat16, y_dtype=torch.float32, path: str = "auto",
              routing: Routing = Routing(), mxfp4: bool = False,
              expert_format: Optional[str] = None, mx_line_rows: bool = False) -> MoeDesc:
    """Layer descriptor.  ``expert_format``: None / "dense", "mxfp4" or
    "mxfp8" (``mxfp4=True`` is the same as "mxfp4").  ``mx_line_rows``: MX
    code rows padded to whole 128-byte lines (MOE_FLAG_MX_LINE_ROWS)."""
    fmt = expert_format or ("mxfp4" if mxfp4 else "dense")
    return MoeDesc(T=T, d=d, E=E, k=k, ffn=ffn, n_shared=n_shared,
                   ffn_shared=ffn_shared if n_shared else 0, dtype=_DT[dtype],
                   y_dtype=_DT[y_dtype], path=_PATHS[path], scoring=_SCORING[routing.scoring],
                   weighting=_lib.WEIGHTS_RENORM if routing.renormalize else _lib.WEIGHTS_RAW,
                   expert_format={"dense": _lib.EXPERTS_DENSE, "mxfp4": _lib.EXPERTS_MXFP4,
                                  "mxfp8": _lib.EXPERTS_MXFP8}[fmt],
                   flags=_lib.FLAG_MX_LINE_ROWS if mx_line_rows else 0,
                   capacity_factor=float(routing.capacity_factor))


def _check(status: int, where: str):
    if status != 0:
        raise MoeError(status, where)


def moe_validate(desc: MoeDesc) -> int:
    return _lib.lib().moe_validate(ctypes.byref(desc))


def moe_workspace_size(desc: MoeDesc) -> int:
    n = ctypes.c_size_t(0)
    _check(_lib.lib().moe_workspace_size(ctypes.byref(desc), ctypes.byref(n)),
           "moe_workspace_size")
    return n.value


def moe_resolve_path(desc: MoeDesc) -> str:
    p = _lib.lib().moe_resolve_path(ctypes.byref(desc))
    if p < 0:
        raise MoeError(p, "moe_resolve_path")
    return {v: k for k, v in _PATHS.items()}[p]


def moe_grouped_rows(desc: MoeDesc) -> int:
    r = _lib.lib().moe_grouped_rows(ctypes.byref(desc))
    if r < 0:
        raise MoeError(int(r), "moe_grouped_rows")
    return int(r)


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors must be on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(device) -> ctypes.c_void_p:
    return ctypes.c_void_p(torch.cuda.current_stream(device).cuda_stream)


def workspace(desc: MoeDesc, device) -> torch.Tensor:
    return torch.empty(moe_workspace_size(desc), dtype=torch.uint8, device=device)


@dataclass
class Weights:
    """Stacked layer weights (device tensors in the layer's storage dtype)."""
    w_router: torch.Tensor                 # [E, d]
    w_up: torch.Tensor                     # [E, ffn, d]
    w_gate: torch.Tensor                   # [E, ffn, d]
    w_down: torch.Tensor                   # [E, d, ffn]
    bias: Optional[torch.Tensor] = None    # [E] float32
    ws_up: Optional[torch.Tensor] = None   # [S, ffn_s, d]
    ws_gate: Optional[torch.Tensor] = None
    ws_down: Optional[torch.Tensor] = None  # [S, d, ffn_s]

    def desc(self, T: int, k: int, y_dtype=torch.float32, path: str = "auto",
             routing: Routing = Routing()) -> MoeDesc:
        E, ffn, d = self.w_up.shape
        ns = 0 if self.ws_up is None else self.ws_up.shape[0]
        fs = 0 if self.ws_up is None else self.ws_up.shape[1]
        return make_desc(T, d, E, k, ffn, ns, fs, self.w_up.dtype, y_dtype, path, routing)


def _check_weights(W: Weights, x: torch.Tensor):
    E, ffn, d = W.w_up.shape
    dt = x.dtype
    if dt not in _DT:
        raise ValueError(f"unsupported dtype {dt}")
    for name in ("w_router", "w_up", "w_gate", "w_down", "ws_up", "ws_gate", "ws_down"):
        t = getattr(W, name)
        if t is not None and t.dtype != dt:
            raise ValueError(f"{name} has dtype {t.dtype}, x has {dt}")
    if tuple(W.w_router.shape) != (E, d) or tuple(W.w_gate.shape) != (E, ffn, d) \
            or tuple(W.w_down.shape) != (E, d, ffn) or x.shape[-1] != d:
        raise ValueError("weight shapes do not match")
    if W.bias is not None and (W.bias.dtype != torch.float32 or tuple(W.bias.shape) != (E,)):
        raise ValueError("bias must be float32 [E]")


def moe_forward(x: torch.Tensor, W: Weights, k: int, y_dtype=torch.float32, path: str = "auto",
                ws: Optional[torch.Tensor] = None, return_routing: bool = False,
                routing: Routing = Routing()):
    """y = MoE(x).  With return_routing, also (topk_idx, topk_w, expert_counts)."""
    _check_weights(W, x)
    T = x.shape[0]
    desc = W.desc(T, k, y_dtype, path, routing)
    dev = x.device
    if ws is None:
        ws = workspace(desc, dev)
    y = torch.empty((T, x.shape[1]), dtype=y_dtype, device=dev)
    idx = w = counts = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((W.w_up.shape[0],), dtype=torch.int32, device=dev)
    st = _lib.lib().moe_forward(ctypes.byref(desc), _ptr(x), _ptr(W.w_router), _ptr(W.bias),
                                _ptr(W.w_up), _ptr(W.w_gate), _ptr(W.w_down), _ptr(W.ws_up),
                                _ptr(W.ws_gate), _ptr(W.ws_down), _ptr(y), _ptr(idx), _ptr(w),
                                _ptr(counts), _ptr(ws), ws.numel(), _stream(dev))
    _check(st, "moe_forward")
    return (y, idx, w, counts) if return_routing else y


def moe_forward_noalloc(x: torch.Tensor, W: Weights, k: int, y_dtype=torch.float32,
                        path: str = "auto", return_routing: bool = False,
                        routing: Routing = Routing(), y: Optional[torch.Tensor] = None):
    """moe_forward on the library's own per-GPU scratch (no workspace
    argument; the C call allocates nothing).  Outputs are allocated here
    unless ``y`` is given.  Raises MoeError(MOE_ERR_TOO_LARGE) for layers
    whose workspace exceeds the scratch."""
    _check_weights(W, x)
    T = x.shape[0]
    desc = W.desc(T, k, y_dtype, path, routing)
    dev = x.device
    if y is None:
        y = torch.empty((T, x.shape[1]), dtype=y_dtype, device=dev)
    idx = w = counts = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((W.w_up.shape[0],), dtype=torch.int32, device=dev)
    st = _lib.lib().moe_forward_noalloc(ctypes.byref(desc), _ptr(x), _ptr(W.w_router),
                                        _ptr(W.bias), _ptr(W.w_up), _ptr(W.w_gate),
                                        _ptr(W.w_down), _ptr(W.ws_up), _ptr(W.ws_gate),
                                        _ptr(W.ws_down), _ptr(y), _ptr(idx), _ptr(w),
                                        _ptr(counts), _stream(dev))
    _check(st, "moe_forward_noalloc")
    return (y, idx, w, counts) if return_routing else y


@dataclass
class MxWeights:
    """A layer whose expert weights are MX-format: MXFP4 (uint8 E2M1 code
    tensors, two codes per byte, element 2i in the low nibble) or MXFP8 (one
    E4M3 code per byte), with uint8 E8M0 scale tensors (one per 32 elements
    along K).  The format follows from the code tensors' last dimension.
    Router weight (bf16) and bias as in ``Weights``."""
    w_router: torch.Tensor                 # [E, d] bf16
    up: torch.Tensor                       # [E, ffn, d/2] (MXFP4) or [E, ffn, d] (MXFP8) uint8
    up_scale: torch.Tensor                 # [E, ffn, d/32] uint8
    gate: torch.Tensor
    gate_scale: torch.Tensor
    down: torch.Tensor                     # [E, d, ffn/2] or [E, d, ffn] uint8
    down_scale: torch.Tensor               # [E, d, ffn/32] uint8
    bias: Optional[torch.Tensor] = None    # [E] float32
    s_up: Optional[torch.Tensor] = None    # shared experts, same layout with ffn_shared
    s_up_scale: Optional[torch.Tensor] = None
    s_gate: Optional[torch.Tensor] = None
    s_gate_scale: Optional[torch.Tensor] = None
    s_down: Optional[torch.Tensor] = None
    s_down_scale: Optional[torch.Tensor] = None
    # code rows padded to whole 128-byte lines: the code tensors' last
    # dimension is the row's code bytes rounded up to a multiple of 128
    line_rows: bool = False
    # "mxfp4" or "mxfp8"; None: from the code tensors' last dimension (which
    # is ambiguous only for padded rows of d <= 128)
    expert_format: Optional[str] = None

    @property
    def format(self) -> str:
        if self.expert_format is not None:
            return self.expert_format
        d = self.up_scale.shape[2] * 32
        return "mxfp8" if self.up.shape[2] == _row_bytes(d, 1, self.line_rows) else "mxfp4"

    def desc(self, T: int, k: int, y_dtype=torch.float32,
             routing: Routing = Routing()) -> MoeDesc:
        E, ffn, _ = self.up.shape
        d = self.up_scale.shape[2] * 32
        ns = 0 if self.s_up is None else self.s_up.shape[0]
        fs = 0 if self.s_up is None else self.s_up.shape[1]
        return make_desc(T, d, E, k, ffn, ns, fs, torch.bfloat16, y_dtype, "auto",
                         routing, expert_format=self.format, mx_line_rows=self.line_rows)


def _row_bytes(K: int, per: int, line_rows: bool) -> int:
    """Bytes of one code row of K codes, `per` codes per byte (rounded up to
    whole 128-byte lines with line_rows)."""
    n = K // per
    return (n + 127) // 128 * 128 if line_rows else n


def _check_mx(W: MxWeights, x: torch.Tensor):
    E, ffn, _ = W.up.shape
    d = W.up_scale.shape[2] * 32
    per = 2 if W.format == "mxfp4" else 1   # codes per byte
    if x.dtype != torch.bfloat16 or W.w_router.dtype != torch.bfloat16:
        raise ValueError("MX-format layers take bf16 x and router weight")
    rb = lambda K: _row_bytes(K, per, W.line_rows)
    want = {"up": (E, ffn, rb(d)), "gate": (E, ffn, rb(d)), "down": (E, d, rb(ffn)),
            "up_scale": (E, ffn, d // 32), "gate_scale": (E, ffn, d // 32),
            "down_scale": (E, d, ffn // 32)}
    for name, shape in want.items():
        t = getattr(W, name)
        if t.dtype != torch.uint8 or tuple(t.shape) != shape:
            raise ValueError(f"{name} must be uint8 {shape}")
    if tuple(W.w_router.shape) != (E, d) or x.shape[-1] != d:
        raise ValueError("router weight or x does not match the experts")
    if W.bias is not None and (W.bias.dtype != torch.float32 or tuple(W.bias.shape) != (E,)):
        raise ValueError("bias must be float32 [E]")


def moe_forward_mx(x: torch.Tensor, W: MxWeights, k: int, y_dtype=torch.float32,
                   ws: Optional[torch.Tensor] = None, return_routing: bool = False,
                   routing: Routing = Routing(), events=None, y: Optional[torch.Tensor] = None):
    """y = MoE(x) with MX-format (MXFP4 or MXFP8) expert weights.  With return_routing, also
    (topk_idx, topk_w, expert_counts).  ``events``: a void** of 6 hipEvents
    (see moe_forward_timed) or None; ``y``: a preallocated output."""
    _check_mx(W, x)
    T = x.shape[0]
    desc = W.desc(T, k, y_dtype, routing)
    dev = x.device
    if ws is None:
        ws = workspace(desc, dev)
    if y is None:
        y = torch.empty((T, x.shape[1]), dtype=y_dtype, device=dev)
    idx = w = counts = None
    if return_routing:
        idx = torch.empty((T, k), dtype=torch.int32, device=dev)
        w = torch.empty((T, k), dtype=torch.float32, device=dev)
        counts = torch.empty((W.up.shape[0],), dtype=torch.int32, device=dev)
    sc = _lib.MoeMxScales(_ptr(W.up_scale), _ptr(W.gate_scale), _ptr(W.down_scale),
                          _ptr(W.s_up_scale), _ptr(W.s_gate_scale), _ptr(W.s_down_scale))
    st = _lib.lib().moe_forward_mx(ctypes.byref(desc), _ptr(x), _ptr(W.w_router), _ptr(W.bias),
                                   _ptr(W.up), _ptr(W.gate), _ptr(W.down), _ptr(W.s_up),
                                   _ptr(W.s_gate), _ptr(W.s_down), ctypes.byref(sc), _ptr(y),
                                   _ptr(idx), _ptr(w), _ptr(counts), _ptr(ws), ws.numel(),
                                   _stream(dev), events)
    _check(st, "moe_forward_mx")
    return (y, idx, w, counts) if return_routing else y


def moe_forward_timed(x: torch.Tensor, W: Weights, k: int, events, y: torch.Tensor,
                      ws: torch.Tensor, y_dtype=torch.float32, path: str = "auto",
                      counts: Optional[torch.Tensor] = None,
                      routing: Routing = Routing()) -> None:
    """moe_forward into preallocated y/ws, recording the 6 hipEvents at
    ``events`` (a void** from hipevents.Events.slice) around its launches."""
    T = x.shape[0]
    desc = W.desc(T, k, y_dtype, path, routing)
    st = _lib.lib().moe_forward_timed(ctypes.byref(desc), _ptr(x), _ptr(W.w_router),
                                      _ptr(W.bias), _ptr(W.w_up), _ptr(W.w_gate),
                                      _ptr(W.w_down), _ptr(W.ws_up), _ptr(W.ws_gate),
                                      _ptr(W.ws_down), _ptr(y), None, None, _ptr(counts),
                                      _ptr(ws), ws.numel(), _stream(x.device), events)
    _check(st, "moe_forward_timed")


def moe_route(x: torch.Tensor, W: Weights, k: int, ws: Optional[torch.Tensor] = None,
              routing: Routing = Routing()):
    """(topk_idx [T,k] int32, topk_w [T,k] float32)."""
    _check_weights(W, x)
    T = x.shape[0]
    desc = W.desc(T, k, routing=routing)
    dev = x.device
    ws = workspace(desc, dev) if ws is None else ws
    idx = torch.empty((T, k), dtype=torch.int32, device=dev)
    w = torch.empty((T, k), dtype=torch.float32, device=dev)
    _check(_lib.lib().moe_route(ctypes.byref(desc), _ptr(x), _ptr(W.w_router), _ptr(W.bias),
                                _ptr(idx), _ptr(w), _ptr(ws), ws.numel(), _stream(dev)),
           "moe_route")
    return idx, w


def moe_dispatch(desc: MoeDesc, topk_idx: torch.Tensor, ws: Optional[torch.Tensor] = None):
    """(expert_counts [E], group_offsets [G+1], sorted_token [R], slot_row [T,k])."""
    dev = topk_idx.device
    if topk_idx.dtype != torch.int32 or tuple(topk_idx.shape) != (desc.T, desc.k):
        raise ValueError("topk_idx must be int32 [T,k]")
    ws = workspace(desc, dev) if ws is None else ws
    R = moe_grouped_rows(desc)
    counts = torch.empty((desc.E,), dtype=torch.int32, device=dev)
    offsets = torch.empty((desc.E + desc.n_shared + 1,), dtype=torch.int32, device=dev)
    sorted_token = torch.empty((R,), dtype=torch.int32, device=dev)
    slot_row = torch.empty((desc.T, desc.k), dtype=torch.int32, device=dev)
    _check(_lib.lib().moe_dispatch(ctypes.byref(desc), _ptr(topk_idx), _ptr(counts),
                                   _ptr(offsets), _ptr(sorted_token), _ptr(slot_row), _ptr(ws),
                                   ws.numel(), _stream(dev)), "moe_dispatch")
    return counts, offsets, sorted_token, slot_row


def moe_experts(x: torch.Tensor, W: Weights, k: int, group_offsets: torch.Tensor,
                sorted_token: torch.Tensor, path: str = "auto",
                ws: Optional[torch.Tensor] = None) -> torch.Tensor:
    """expert_out [R, d] float32: FFN of each grouped row's group."""
    _check_weights(W, x)
    desc = W.desc(x.shape[0], k, path=path)
    dev = x.device
    ws = workspace(desc, dev) if ws is None else ws
    R = moe_grouped_rows(desc)
    if group_offsets.dtype != torch.int32 or sorted_token.dtype != torch.int32 \
            or group_offsets.numel() != desc.E + desc.n_shared + 1 or sorted_token.numel() != R:
        raise ValueError("group_offsets / sorted_token do not match the layer")
    out = torch.empty((R, x.shape[1]), dtype=torch.float32, device=dev)
    _check(_lib.lib().moe_experts(ctypes.byref(desc), _ptr(x), _ptr(W.w_up), _ptr(W.w_gate),
                                  _ptr(W.w_down), _ptr(W.ws_up), _ptr(W.ws_gate),
                                  _ptr(W.ws_down), _ptr(group_offsets), _ptr(sorted_token),
                                  _ptr(out), _ptr(ws), ws.numel(), _stream(dev)), "moe_experts")
    return out


def moe_combine(desc: MoeDesc, expert_out: torch.Tensor, topk_w: torch.Tensor,
                slot_row: torch.Tensor, group_offsets: torch.Tensor,
                y_dtype=torch.float32) -> torch.Tensor:
    """y [T, d] from the expert outputs."""
    dev = expert_out.device
    if expert_out.dtype != torch.float32 or topk_w.dtype != torch.float32:
        raise ValueError("expert_out and topk_w must be float32")
    y = torch.empty((desc.T, desc.d), dtype=y_dtype, device=dev)
    _check(_lib.lib().moe_combine(ctypes.byref(desc), _ptr(expert_out), _ptr(topk_w),
                                  _ptr(slot_row), _ptr(group_offsets), _ptr(y), _stream(dev)),
           "moe_combine")
    return y
