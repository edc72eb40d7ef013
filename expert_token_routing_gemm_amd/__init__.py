"""MI355X-native MoE-layer forward (route -> dispatch -> expert FFN ->
combine) on one GPU's share of the work.

Thin Python binding over the C ABI of ``libmoe.so`` (include/moe.h): the
functions below only marshal torch tensors (device memory) and the current
HIP stream into the C argument structures.  Every step of the layer runs in
the library's HIP kernels; there is no Python or CPU fallback.

``MoELayer`` holds the device buffers of one workload (inputs uploaded from
host arrays, outputs and workspace sized from the shapes) and the filled-in
``moe_layer_args`` so that a forward is a single C call.
"""
from __future__ import annotations

import ctypes as C
from typing import Optional

import numpy as np
import torch

from . import _abi
from ._abi import (INT32_MAX, MOE_BF16, MOE_F32, MOE_FP8_E4M3, MOE_GELU, MOE_LAYER_EVENTS,  # noqa: F401
                   MOE_STATIC_SCRATCH_BYTES, MOE_RELU, MOE_SIGMOID, MOE_SOFTMAX, MOE_SWIGLU, MOE_W_ROWMAJOR, MOE_W_TILED16,
                   CombineArgs, DispatchArgs,
                   FfnArgs, LayerArgs, RouteArgs, lib)

DTYPE = {"f32": MOE_F32, "bf16": MOE_BF16, "fp8": MOE_FP8_E4M3}
SCORE = {"softmax": MOE_SOFTMAX, "sigmoid": MOE_SIGMOID}
ACT = {"relu": MOE_RELU, "gelu": MOE_GELU, "swiglu": MOE_SWIGLU}


class MoEError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what} failed with status {status}: {lib().moe_last_error().decode()}")
        self.status = status


def _check(status: int, what: str) -> None:
    if status != 0:
        raise MoEError(status, what)


def _p(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream=None) -> int:
    s = stream if stream is not None else torch.cuda.current_stream()
    return s.cuda_stream


def _used_on(stream, *tensors) -> None:
    """Temporaries allocated on the current stream but read by work on
    ``stream``: keep the caching allocator from reusing them before it ends."""
    if stream is not None:
        for t in tensors:
            t.record_stream(stream)


# ------------------------------------------------------------ host helpers


def moe_capacity(T: int, k: int, E: int, cf: Optional[float]) -> int:
    """ceil(cf*T*k/E) computed by the library; None/<=0 -> no limit."""
    return int(lib().moe_capacity(T, k, E, 0.0 if cf is None else float(cf)))


def moe_send_rows_max(T: int, k: int, E: int, capacity: int) -> int:
    return int(lib().moe_send_rows_max(T, k, E, capacity))


def moe_route_workspace_bytes(a: RouteArgs) -> int:
    return int(lib().moe_route_workspace_bytes(C.byref(a)))


def moe_dispatch_workspace_bytes(a: DispatchArgs) -> int:
    return int(lib().moe_dispatch_workspace_bytes(C.byref(a)))


def moe_ffn_workspace_bytes(a: FfnArgs) -> int:
    return int(lib().moe_ffn_workspace_bytes(C.byref(a)))


def moe_workspace_bytes(a: LayerArgs) -> int:
    return int(lib().moe_workspace_bytes(C.byref(a)))


# ------------------------------------------------------------ entry points


def moe_route(a: RouteArgs, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_route(C.byref(a), _p(workspace), ws_bytes, _stream(stream)), "moe_route")


def moe_dispatch(a: DispatchArgs, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_dispatch(C.byref(a), _p(workspace), ws_bytes, _stream(stream)), "moe_dispatch")


def moe_expert_ffn(a: FfnArgs, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_expert_ffn(C.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "moe_expert_ffn")


def moe_combine(a: CombineArgs, stream=None) -> None:
    _check(lib().moe_combine(C.byref(a), _stream(stream)), "moe_combine")


def moe_bias_update(counts: torch.Tensor, b_select: torch.Tensor, T: int, k: int, gamma: float,
                    stream=None) -> None:
    """In-place bias-balancing step on device tensors counts [E] (int32) and
    b_select [E] (float32)."""
    _check(lib().moe_bias_update(_p(counts), _p(b_select), int(counts.numel()), int(T), int(k),
                                 float(gamma), _stream(stream)), "moe_bias_update")


def moe_aux_loss(logits: torch.Tensor, counts: torch.Tensor, k: int, score: int, alpha: float,
                 stream=None):
    """Auxiliary balancing loss of one step: (prob_mean [E], loss [1]) device
    tensors from the router's fp32 logits [T, E] and the raw counts [E]."""
    T, E = logits.shape
    ws = torch.empty((max(int(lib().moe_aux_loss_workspace_bytes(T, E)), 256),), dtype=torch.uint8,
                     device=logits.device)
    pm = torch.empty((E,), dtype=torch.float32, device=logits.device)
    loss = torch.empty((1,), dtype=torch.float32, device=logits.device)
    _check(lib().moe_aux_loss(_p(logits), _p(counts), int(T), int(E), int(k), int(score),
                              float(alpha), _p(pm), _p(loss), _p(ws), ws.numel(), _stream(stream)),
           "moe_aux_loss")
    _used_on(stream, ws, pm, loss)
    return pm, loss


def moe_weight_tile(w: torch.Tensor, n_mats: int, rows: int, stream=None) -> torch.Tensor:
    """A new device tensor holding the n_mats [rows, *] matrices of ``w``
    (contiguous) in the 16-row tiled layout of the streaming kernels."""
    w = w.contiguous()
    out = torch.empty_like(w)
    nbytes = w.numel() * w.element_size()
    row_bytes = nbytes // max(1, n_mats * rows)
    _check(lib().moe_weight_tile(_p(w), _p(out), int(n_mats), int(rows), int(row_bytes),
                                 _stream(stream)), "moe_weight_tile")
    _used_on(stream, w, out)
    return out


def moe_layer_forward(a: LayerArgs, workspace: Optional[torch.Tensor], stream=None) -> None:
    ws_bytes = 0 if workspace is None else workspace.numel() * workspace.element_size()
    _check(lib().moe_layer_forward(C.byref(a), _p(workspace), ws_bytes, _stream(stream)),
           "moe_layer_forward")


def moe_layer_forward_noalloc(a: LayerArgs, stream=None) -> None:
    """The layer forward on the library's static scratch (no workspace)."""
    _check(lib().moe_layer_forward_noalloc(C.byref(a), _stream(stream)),
           "moe_layer_forward_noalloc")


# ------------------------------------------------------------ buffers


def to_device(arr: Optional[np.ndarray], device="cuda") -> Optional[torch.Tensor]:
    """Host array -> device tensor with the same bytes (bf16 bit patterns as
    torch.bfloat16, fp8 bytes as torch.uint8)."""
    if arr is None:
        return None
    arr = np.ascontiguousarray(arr)
    if arr.dtype == np.uint16:
        t = torch.from_numpy(arr.view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(arr)
    return t.to(device)


def to_host(t: torch.Tensor) -> np.ndarray:
    """Device tensor -> numpy (bf16 as uint16 bit patterns)."""
    t = t.detach().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


class MoELayer:
    """Device state of one MoE layer workload.

    ``wl`` is any object with the attributes of ``synth.Workload`` (shapes,
    dtype tags, host arrays).  ``capacity`` overrides the capacity computed
    from ``wl.cf``; ``logits_input`` (fp32 [T, E] host array) switches route
    to the identical-logits mode."""

    def __init__(self, wl, device="cuda", capacity: Optional[int] = None,
                 logits_input: Optional[np.ndarray] = None, keep_logits: bool = True,
                 n_groups: int = 0, topk_groups: int = 0, w_layout: int = 0):
        self.wl = wl
        dev = torch.device(device)
        self.device = dev
        T, d, E, k, R, h = wl.T, wl.d, wl.E, wl.k, wl.R, wl.h
        self.T, self.k = T, k
        self.act_dtype = DTYPE[wl.act_dtype]
        tdt = torch.float32 if wl.act_dtype == "f32" else torch.bfloat16
        self.capacity = moe_capacity(T, k, E, wl.cf) if capacity is None else int(capacity)
        self.rows_max = moe_send_rows_max(T, k, E, self.capacity)
        nx = wl.e_end - wl.e_begin
        self.ffn_rows = min(self.rows_max, nx * min(T, self.capacity))
        i32 = dict(dtype=torch.int32, device=dev)
        f32 = dict(dtype=torch.float32, device=dev)
        # inputs
        self.x = to_device(wl.x, dev)
        self.w_router = to_device(wl.w_router, dev)
        self.b_router = to_device(wl.b_router, dev)
        self.b_select = to_device(wl.b_select, dev)
        self.w1, self.w3, self.w2 = (to_device(wl.w1, dev), to_device(wl.w3, dev),
                                     to_device(wl.w2, dev))
        self.s1, self.s3, self.s2 = (to_device(wl.s1, dev), to_device(wl.s3, dev),
                                     to_device(wl.s2, dev))
        sh = wl.shared or {}
        self.ws1, self.ws3, self.ws2 = (to_device(sh.get("w1"), dev), to_device(sh.get("w3"), dev),
                                        to_device(sh.get("w2"), dev))
        self.w_layout = int(w_layout)
        if self.w_layout == _abi.MOE_W_TILED16:
            nx = wl.e_end - wl.e_begin
            til = lambda w, n, r: None if w is None else moe_weight_tile(w, n, r)  # noqa: E731
            self.w1, self.w3, self.w2 = til(self.w1, nx, h), til(self.w3, nx, h), til(self.w2, nx, d)
            self.ws1, self.ws3, self.ws2 = (til(self.ws1, 1, h), til(self.ws3, 1, h),
                                            til(self.ws2, 1, d))
        self.ss1, self.ss3, self.ss2 = (to_device(sh.get("s1"), dev), to_device(sh.get("s3"), dev),
                                        to_device(sh.get("s2"), dev))
        # outputs
        self.identical_logits = logits_input is not None
        if self.identical_logits:
            self.logits = to_device(np.ascontiguousarray(logits_input, np.float32), dev)
        else:
            self.logits = torch.empty((T, E), **f32) if keep_logits else None
        self.ids = torch.empty((T, k), **i32)
        self.weights = torch.empty((T, k), **f32)
        self.counts = torch.empty((E,), **i32)
        self.kept = torch.empty((E,), **i32)
        self.expert_off = torch.empty((E + 1,), **i32)
        self.rank_counts = torch.empty((R,), **i32)
        self.rank_off = torch.empty((R + 1,), **i32)
        self.slot = torch.empty((T, k), **i32)
        self.src = torch.empty((max(self.rows_max, 1),), **i32)
        self.x_send = torch.empty((max(self.rows_max, 1), d), dtype=tdt, device=dev)
        self.y_send = torch.empty((max(self.rows_max, 1), d), dtype=tdt, device=dev)
        self.y_dense = torch.empty((T, d), dtype=tdt, device=dev) if wl.shared else None
        self.y = torch.empty((T, d), dtype=tdt, device=dev)

        a = LayerArgs()
        r = a.route
        r.T, r.d, r.E, r.k = T, d, E, k
        r.act_dtype, r.score, r.renorm = self.act_dtype, SCORE[wl.score], int(bool(wl.renorm))
        r.n_groups, r.topk_groups = int(n_groups), int(topk_groups)
        r.x = None if self.identical_logits else _p(self.x)
        r.w_router = _p(self.w_router)
        r.b_router = None if self.identical_logits else _p(self.b_router)
        r.b_select = _p(self.b_select)
        r.logits, r.ids, r.weights = _p(self.logits), _p(self.ids), _p(self.weights)
        ds = a.dispatch
        ds.T, ds.d, ds.E, ds.k, ds.R = T, d, E, k, R
        ds.capacity, ds.act_dtype = self.capacity, self.act_dtype
        ds.ids, ds.x = _p(self.ids), _p(self.x)
        ds.counts, ds.kept, ds.expert_off = _p(self.counts), _p(self.kept), _p(self.expert_off)
        ds.rank_counts, ds.rank_off = _p(self.rank_counts), _p(self.rank_off)
        ds.slot, ds.src, ds.x_send = _p(self.slot), _p(self.src), _p(self.x_send)
        f = a.ffn
        f.d, f.h, f.E, f.e_begin, f.e_end = d, h, E, wl.e_begin, wl.e_end
        f.act, f.act_dtype, f.w_dtype = ACT[wl.act], self.act_dtype, DTYPE[wl.w_dtype]
        f.w_layout = self.w_layout
        f.max_rows = self.ffn_rows
        f.x_send, f.expert_off = _p(self.x_send), _p(self.expert_off)
        f.w1, f.w3, f.w2 = _p(self.w1), _p(self.w3), _p(self.w2)
        f.s1, f.s3, f.s2 = _p(self.s1), _p(self.s3), _p(self.s2)
        f.y_send = _p(self.y_send)
        if wl.shared:
            f.T_dense, f.x_dense = T, _p(self.x)
            f.ws1, f.ws3, f.ws2 = _p(self.ws1), _p(self.ws3), _p(self.ws2)
            f.ss1, f.ss3, f.ss2 = _p(self.ss1), _p(self.ss3), _p(self.ss2)
            f.y_dense = _p(self.y_dense)
        c = a.combine
        c.T, c.d, c.k, c.e_begin, c.e_end = T, d, k, wl.e_begin, wl.e_end
        c.act_dtype = self.act_dtype
        c.x, c.shared_out, c.y_send = _p(self.x), _p(self.y_dense), _p(self.y_send)
        c.ids, c.slot, c.weights, c.y = _p(self.ids), _p(self.slot), _p(self.weights), _p(self.y)
        self.args = a
        nbytes = max(moe_workspace_bytes(a), 256)
        self.workspace = torch.empty((nbytes,), dtype=torch.uint8, device=dev)

    # single stages (each one C call)
    def aux_loss(self, alpha: float, stream=None):
        """Auxiliary balancing loss of the last route + dispatch (needs the
        logits kept): (prob_mean [E], loss [1]) device tensors."""
        if self.logits is None:
            raise ValueError("the layer does not keep its logits")
        return moe_aux_loss(self.logits, self.counts, self.k, SCORE[self.wl.score], alpha, stream)

    def update_bias(self, gamma: float, stream=None) -> None:
        """One bias-balancing step from the last dispatch's raw counts."""
        if self.b_select is None:
            raise ValueError("the workload has no selection bias")
        moe_bias_update(self.counts, self.b_select, self.T, self.k, gamma, stream)

    def route(self, stream=None):
        moe_route(self.args.route, self.workspace, stream)

    def dispatch(self, stream=None):
        moe_dispatch(self.args.dispatch, self.workspace, stream)

    def expert_ffn(self, stream=None):
        moe_expert_ffn(self.args.ffn, self.workspace, stream)

    def combine(self, stream=None):
        moe_combine(self.args.combine, stream)

    def forward(self, events=None, stream=None):
        """Whole layer; ``events`` = list of MOE_LAYER_EVENTS raw hipEvent_t
        handles (ints; None skips that boundary) recorded at the stage
        boundaries, or None."""
        self._set_events(events)
        moe_layer_forward(self.args, self.workspace, stream)

    def _set_events(self, events):
        if events is not None:
            arr = (C.c_void_p * MOE_LAYER_EVENTS)(*events)
            self.args.events = C.cast(arr, C.POINTER(C.c_void_p))
            self._ev_keep = arr
        else:
            self.args.events = None

    def forward_noalloc(self, events=None, stream=None):
        """Whole layer through the no-allocation entry point (the library's
        static scratch instead of this layer's workspace)."""
        self._set_events(events)
        moe_layer_forward_noalloc(self.args, stream)

    def results(self) -> dict:
        torch.cuda.synchronize(self.device)
        out = dict(ids=to_host(self.ids), weights=to_host(self.weights),
                   counts=to_host(self.counts), kept=to_host(self.kept),
                   off=to_host(self.expert_off), rank_counts=to_host(self.rank_counts),
                   rank_off=to_host(self.rank_off), slot=to_host(self.slot))
        n = int(out["off"][-1])
        out["src"] = to_host(self.src[:n])
        if self.logits is not None:
            out["logits"] = to_host(self.logits)
        return out
