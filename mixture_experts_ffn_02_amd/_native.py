"""ctypes declarations of libmoe.so (the C ABI in include/moe.h).

Argument marshalling only: every step of the layer runs in the library's HIP
kernels. Loading fails loudly when the library has not been built.
"""
from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmoe.so")

MOE_F32, MOE_BF16 = 0, 1
MOE_SOFTMAX, MOE_SIGMOID = 0, 1
MOE_N_PHASES = 8
PHASES = ("route", "scan", "scatter", "gateup", "down", "shared_gateup", "shared_down", "combine")
MOE_N_METRICS = 6
METRICS = ("z_loss", "aux_loss", "cv", "entropy_bits", "load_max_ratio", "unused_frac")

STATUS = {0: "MOE_OK", 1: "MOE_ERR_INVALID", 2: "MOE_ERR_UNSUPPORTED", 3: "MOE_ERR_WORKSPACE", 4: "MOE_ERR_HIP"}

# Every symbol include/moe.h declares.
EXPORTS = (
    "moe_status_str", "moe_workspace_size", "moe_route", "moe_route_ex", "moe_bias_update", "moe_permute",
    "moe_grouped_swiglu_workspace_size", "moe_grouped_swiglu", "moe_combine", "moe_forward", "moe_forward_ex",
    "moe_timing_create", "moe_timing_destroy", "moe_timing_read", "moe_timing_select", "moe_backward_workspace_size", "moe_backward",
    "moe_forward_noalloc",
)
# Bytes of the library's fixed scratch array used by moe_forward_noalloc.
MOE_NOALLOC_BYTES = 256 << 20


class MoeError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: {STATUS.get(status, status)}")
        self.status = status


class MoeLayerC(ctypes.Structure):
    _fields_ = [
        ("d_model", ctypes.c_int32), ("d_ff", ctypes.c_int32), ("n_experts", ctypes.c_int32),
        ("top_k", ctypes.c_int32), ("score", ctypes.c_int32), ("renorm", ctypes.c_int32),
        ("dtype", ctypes.c_int32), ("d_ff_shared", ctypes.c_int32), ("bias_on_logits", ctypes.c_int32),
        ("w_router", ctypes.c_void_p), ("sel_bias", ctypes.c_void_p),
        ("w_gate", ctypes.c_void_p), ("w_up", ctypes.c_void_p), ("w_down", ctypes.c_void_p),
        ("ws_gate", ctypes.c_void_p), ("ws_up", ctypes.c_void_p), ("ws_down", ctypes.c_void_p),
    ]


class MoeRouteOptsC(ctypes.Structure):
    _fields_ = [("sel_noise", ctypes.c_void_p), ("metrics", ctypes.c_void_p)]


class MoeGradsC(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("dx", "dw_router", "dw_gate", "dw_up", "dw_down", "dws_gate", "dws_up",
                                               "dws_down", "d_topk_w")]


_lib = None


def load(path: str = LIB_PATH) -> ctypes.CDLL:
    global _lib
    if _lib is not None and path == LIB_PATH:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is not built; run `python -m mixture_experts_ffn_02_amd.build`")
    L = ctypes.CDLL(path)
    vp, i32, i64, sz = ctypes.c_void_p, ctypes.c_int32, ctypes.c_int64, ctypes.c_size_t
    P = ctypes.POINTER
    LP = P(MoeLayerC)
    L.moe_status_str.restype = ctypes.c_char_p
    L.moe_status_str.argtypes = [ctypes.c_int]
    L.moe_workspace_size.argtypes = [LP, i64, P(sz)]
    OP = P(MoeRouteOptsC)
    L.moe_route.argtypes = [LP, vp, i64, vp, vp, vp, vp, sz, vp]
    L.moe_route_ex.argtypes = [LP, vp, i64, OP, vp, vp, vp, vp, sz, vp]
    L.moe_bias_update.argtypes = [i32, vp, ctypes.c_float, vp, vp]
    L.moe_permute.argtypes = [LP, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    L.moe_grouped_swiglu_workspace_size.argtypes = [i32, i32, i32, i32, i64, P(sz)]
    L.moe_grouped_swiglu.argtypes = [i32, i32, i32, i32, i64, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.moe_combine.argtypes = [LP, i64, vp, vp, vp, vp, vp, vp]
    L.moe_forward.argtypes = [LP, vp, i64, vp, vp, vp, vp, vp, sz, vp]
    L.moe_timing_create.argtypes = [P(vp)]
    L.moe_timing_destroy.argtypes = [vp]
    L.moe_forward_ex.argtypes = [LP, vp, i64, OP, vp, vp, vp, vp, vp, sz, vp, vp]
    L.moe_forward_noalloc.argtypes = [LP, vp, i64, vp, vp, vp, vp, vp]
    L.moe_timing_read.argtypes = [vp, P(ctypes.c_float)]
    L.moe_timing_select.argtypes = [vp, ctypes.c_uint32]
    L.moe_backward_workspace_size.argtypes = [LP, i64, P(sz)]
    L.moe_backward.argtypes = [LP, vp, i64, vp, vp, vp, ctypes.c_float, ctypes.c_float, P(MoeGradsC), vp, sz, vp]
    for name in EXPORTS:
        if name != "moe_status_str":
            getattr(L, name).restype = ctypes.c_int
    if path == LIB_PATH:
        _lib = L
    return L


def check(status: int, what: str) -> None:
    if status != 0:
        raise MoeError(status, what)
