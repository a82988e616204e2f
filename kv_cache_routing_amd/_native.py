"""ctypes view of libsinkroute's C ABI (include/sinkroute.h).

Loads the in-tree kv_cache_routing_amd/libsinkroute.so; there is no fallback:
if the library is missing the import of the binding fails loudly.
"""
from __future__ import annotations

import ctypes
import os

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libsinkroute.so")

SR_OK, SR_ERR_INVALID_ARG, SR_ERR_UNSUPPORTED, SR_ERR_HIP = 0, 1, 2, 3
SR_KV_BF16, SR_KV_F32 = 0, 1
SR_KERNEL_AUTO, SR_KERNEL_VALU, SR_KERNEL_MFMA = 0, 1, 2
SR_READ_BLOCKED, SR_READ_NONTEMPORAL, SR_READ_LDS = 1, 2, 4

# Every function include/sinkroute.h declares.
EXPORTS = (
    "sr_record_sink", "sr_route", "sr_workspace_bytes", "sr_workspace_init",
    "sr_decode_attn", "sr_dense_decode", "sr_splits_for", "sr_split_cap", "sr_grid_size",
    "sr_status_string", "sr_version", "sr_stream_read", "sr_route_decode",
    "sr_dense_decode_alpha0", "sr_rope_append", "sr_plan_parts", "sr_rope_route_decode",
    "sr_route_decode_static",
)
SR_STATIC_SCRATCH_BYTES = 16 << 20


class SrShape(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("seq_len", ctypes.c_int64), ("stride_b", ctypes.c_int64),
        ("stride_h", ctypes.c_int64), ("stride_t", ctypes.c_int64),
        ("kv_dtype", ctypes.c_int32), ("reserved", ctypes.c_int32),
    ]


class SrLaunch(ctypes.Structure):
    _fields_ = [
        ("num_splits", ctypes.c_int32), ("kernel", ctypes.c_int32),
        ("wgs_per_cu", ctypes.c_int32), ("waves_per_wg", ctypes.c_int32),
    ]


class SrPart(ctypes.Structure):
    _fields_ = [
        ("item", ctypes.c_int32), ("part", ctypes.c_int32), ("parts", ctypes.c_int32),
        ("lanes", ctypes.c_int32), ("first", ctypes.c_int64), ("end", ctypes.c_int64),
        ("chunk", ctypes.c_int64),
    ]


class SinkRouteError(RuntimeError):
    def __init__(self, status: int, call: str):
        self.status = status
        super().__init__(f"{call}: {status_string(status)} (status {status})")


def _load():
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with `python kv_cache_routing_amd/build.py` "
            "(or __graft_entry__.build())")
    lib = ctypes.CDLL(LIB_PATH)
    P = ctypes.c_void_p
    S = ctypes.POINTER(SrShape)
    Lp = ctypes.POINTER(SrLaunch)
    i32, f32, sz = ctypes.c_int32, ctypes.c_float, ctypes.c_size_t
    sig = {
        "sr_record_sink": (i32, [S, P, P, P, P, P]),
        "sr_route": (i32, [S, P, P, f32, P, P, P, P, P]),
        "sr_workspace_bytes": (sz, [S, Lp]),
        "sr_workspace_init": (i32, [P, sz, P]),
        "sr_decode_attn": (i32, [S, Lp, P, P, P, P, P, P, f32, P, sz, P, P]),
        "sr_dense_decode": (i32, [S, Lp, P, P, P, f32, P, sz, P, P]),
        "sr_route_decode": (i32, [S, Lp, P, P, P, P, P, f32, f32, P, P, P, P, P, sz, P, P]),
        "sr_route_decode_static": (i32, [S, Lp, P, P, P, P, P, f32, f32, P, P, P, P, P, P]),
        "sr_dense_decode_alpha0": (i32, [S, Lp, P, P, P, f32, P, sz, P, P, P]),
        "sr_rope_append": (i32, [S, P, P, P, P, ctypes.c_int64, P, P, P, P]),
        "sr_rope_route_decode": (i32, [S, Lp, P, P, P, P, P, P, P, P, P, f32, f32, P, P, P, P,
                                       P, sz, P, P]),
        "sr_splits_for": (i32, [S, Lp, i32]),
        "sr_split_cap": (i32, [S, Lp]),
        "sr_grid_size": (i32, [S, Lp]),
        "sr_status_string": (ctypes.c_char_p, [i32]),
        "sr_version": (i32, []),
        "sr_stream_read": (i32, [P, sz, i32, i32, i32, P, P]),
        "sr_plan_parts": (i32, [S, Lp, i32, i32, ctypes.POINTER(SrPart), i32]),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    return lib


lib = _load()


def status_string(status: int) -> str:
    return lib.sr_status_string(int(status)).decode()


def check(status: int, call: str) -> None:
    if status != SR_OK:
        raise SinkRouteError(status, call)
