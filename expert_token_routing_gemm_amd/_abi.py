"""ctypes mirror of include/moe.h and loading of the in-tree libmoe.so.

Nothing here computes: it declares the C structures and function
prototypes.  If the library is missing the import fails loudly; there is no
fallback path.
"""
from __future__ import annotations

import ctypes as C
import os

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "libmoe.so")

MOE_OK, MOE_ERR_INVALID, MOE_ERR_UNSUPPORTED, MOE_ERR_WORKSPACE, MOE_ERR_HIP = 0, -1, -2, -3, -4
MOE_F32, MOE_BF16, MOE_FP8_E4M3 = 0, 1, 2
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_RELU, MOE_GELU, MOE_SWIGLU = 0, 1, 2
MOE_W_ROWMAJOR, MOE_W_TILED16 = 0, 1
MOE_MAX_EXPERTS = 256
MOE_MAX_TOPK = 8
MOE_LAYER_EVENTS = 6
MOE_STATIC_SCRATCH_BYTES = 64 << 20
INT32_MAX = 2 ** 31 - 1

vp = C.c_void_p


class RouteArgs(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("act_dtype", C.c_int32), ("score", C.c_int32), ("renorm", C.c_int32),
                ("n_groups", C.c_int32), ("topk_groups", C.c_int32),
                ("x", vp), ("w_router", vp), ("b_router", vp), ("b_select", vp),
                ("logits", vp), ("ids", vp), ("weights", vp)]


class DispatchArgs(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int32), ("E", C.c_int32), ("k", C.c_int32),
                ("R", C.c_int32), ("capacity", C.c_int32), ("act_dtype", C.c_int32),
                ("ids", vp), ("x", vp), ("counts", vp), ("kept", vp), ("expert_off", vp),
                ("rank_counts", vp), ("rank_off", vp), ("slot", vp), ("src", vp),
                ("x_send", vp)]


class FfnArgs(C.Structure):
    _fields_ = [("d", C.c_int32), ("h", C.c_int32), ("E", C.c_int32), ("e_begin", C.c_int32),
                ("e_end", C.c_int32), ("act", C.c_int32), ("act_dtype", C.c_int32),
                ("w_dtype", C.c_int32), ("w_layout", C.c_int32), ("max_rows", C.c_int64),
                ("x_send", vp),
                ("expert_off", vp), ("w1", vp), ("w3", vp), ("w2", vp), ("s1", vp), ("s3", vp),
                ("s2", vp), ("y_send", vp), ("T_dense", C.c_int64), ("x_dense", vp),
                ("ws1", vp), ("ws3", vp), ("ws2", vp), ("ss1", vp), ("ss3", vp), ("ss2", vp),
                ("y_dense", vp)]


class CombineArgs(C.Structure):
    _fields_ = [("T", C.c_int64), ("d", C.c_int32), ("k", C.c_int32), ("e_begin", C.c_int32),
                ("e_end", C.c_int32), ("act_dtype", C.c_int32), ("x", vp), ("shared_out", vp),
                ("y_send", vp), ("ids", vp), ("slot", vp), ("weights", vp), ("y", vp)]


class LayerArgs(C.Structure):
    _fields_ = [("route", RouteArgs), ("dispatch", DispatchArgs), ("ffn", FfnArgs),
                ("combine", CombineArgs), ("events", C.POINTER(vp))]


# name -> (restype, argtypes): every symbol include/moe.h declares
PROTOTYPES = {
    "moe_route_workspace_bytes": (C.c_size_t, [C.POINTER(RouteArgs)]),
    "moe_route": (C.c_int, [C.POINTER(RouteArgs), vp, C.c_size_t, vp]),
    "moe_capacity": (C.c_int32, [C.c_int64, C.c_int32, C.c_int32, C.c_double]),
    "moe_send_rows_max": (C.c_int64, [C.c_int64, C.c_int32, C.c_int32, C.c_int32]),
    "moe_bias_update": (C.c_int, [vp, vp, C.c_int32, C.c_int64, C.c_int32, C.c_float, vp]),
    "moe_aux_loss_workspace_bytes": (C.c_size_t, [C.c_int64, C.c_int32]),
    "moe_aux_loss": (C.c_int, [vp, vp, C.c_int64, C.c_int32, C.c_int32, C.c_int32, C.c_float, vp,
                               vp, vp, C.c_size_t, vp]),
    "moe_dispatch_workspace_bytes": (C.c_size_t, [C.POINTER(DispatchArgs)]),
    "moe_dispatch": (C.c_int, [C.POINTER(DispatchArgs), vp, C.c_size_t, vp]),
    "moe_ffn_workspace_bytes": (C.c_size_t, [C.POINTER(FfnArgs)]),
    "moe_expert_ffn": (C.c_int, [C.POINTER(FfnArgs), vp, C.c_size_t, vp]),
    "moe_weight_tile": (C.c_int, [vp, vp, C.c_int64, C.c_int32, C.c_int64, vp]),
    "moe_combine": (C.c_int, [C.POINTER(CombineArgs), vp]),
    "moe_workspace_bytes": (C.c_size_t, [C.POINTER(LayerArgs)]),
    "moe_layer_forward": (C.c_int, [C.POINTER(LayerArgs), vp, C.c_size_t, vp]),
    "moe_layer_forward_noalloc": (C.c_int, [C.POINTER(LayerArgs), vp]),
    "moe_last_error": (C.c_char_p, []),
}

_LIB = None


def lib() -> C.CDLL:
    """The loaded libmoe.so (raises if it has not been built)."""
    global _LIB
    if _LIB is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"{LIB_PATH} is missing: build it first "
                              "(python -c 'import __graft_entry__ as g; g.build()')")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in PROTOTYPES.items():
            fn = getattr(L, name)
            fn.restype = res
            fn.argtypes = args
        _LIB = L
    return _LIB
