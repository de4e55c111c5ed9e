"""ctypes loader for libdash_attn.so (argument marshalling only).

The library must have been built (``python -m
deterministic_attention_backward_attn_amd.build``); loading fails loudly
otherwise.  There is no fallback implementation.
"""
from __future__ import annotations

import ctypes
import os
import re

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "libdash_attn.so")
HEADER = os.path.join(os.path.dirname(HERE), "include", "dash_attn.h")

STATUS = {
    0: "DASH_OK",
    1: "DASH_ERR_INVALID_ARG",
    2: "DASH_ERR_UNSUPPORTED",
    3: "DASH_ERR_WORKSPACE",
    4: "DASH_ERR_HIP",
    5: "DASH_ERR_SCHEDULE_INVALID",
    6: "DASH_ERR_ORDER_TIMEOUT",
    7: "DASH_ERR_HOST_MEMORY",
}
NOALLOC_SCRATCH_BYTES = 64 << 20   # DASH_NOALLOC_SCRATCH_BYTES
NOALLOC_WORKSPACE = 1               # DASH_NOALLOC_WORKSPACE
SCHEDULES = {"atomic": 0, "naive": 1, "descending": 2, "shift": 3, "auto": 4}
DTYPES = {"f32": 0, "bf16": 1}


class DashError(RuntimeError):
    def __init__(self, code: int, where: str):
        self.code = code
        super().__init__(f"{where}: {STATUS.get(code, code)}")


class Desc(ctypes.Structure):
    _fields_ = [("B", ctypes.c_int32), ("H", ctypes.c_int32), ("N", ctypes.c_int32),
                ("d", ctypes.c_int32), ("dtype", ctypes.c_int32), ("causal", ctypes.c_int32),
                ("softmax_scale", ctypes.c_float), ("window", ctypes.c_int32),
                ("block_size", ctypes.c_int32), ("block_mask", ctypes.c_void_p)]


class Debug(ctypes.Structure):
    _fields_ = [("spin_limit", ctypes.c_uint32), ("jitter_seed", ctypes.c_uint32),
                ("poison_q", ctypes.c_int32), ("partials", ctypes.c_void_p),
                ("kernel_events", ctypes.c_void_p * 2), ("wait_stats", ctypes.c_void_p),
                ("placement", ctypes.c_int32), ("unit_order", ctypes.c_int32),
                ("phase_stats", ctypes.c_void_p), ("layout", ctypes.c_int32)]


_vp = ctypes.c_void_p
_i32 = ctypes.c_int32
_dp = ctypes.POINTER(ctypes.c_double)
_ip = ctypes.POINTER(ctypes.c_int32)

_SIGS = {
    "dash_status_string": (ctypes.c_char_p, [ctypes.c_int]),
    "dash_attn_tile": (_i32, [ctypes.POINTER(Desc)]),
    "dash_attn_bwd_subtile": (_i32, [ctypes.POINTER(Desc)]),
    "dash_attn_fwd": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _vp, _vp, _vp, _vp, _vp]),
    "dash_attn_bwd_preprocess": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _vp, _vp, _vp]),
    "dash_attn_fwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Desc)]),
    "dash_attn_fwd_ws": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _vp, _vp, _vp, _vp, _vp,
                                        ctypes.c_size_t, _vp]),
    "dash_attn_bwd_workspace_size": (ctypes.c_size_t, [ctypes.POINTER(Desc), ctypes.c_int]),
    "dash_attn_bwd": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, _vp, _vp, _vp, _vp, _vp,
                                     _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _vp]),
    "dash_attn_bwd_debug": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, _vp, _vp, _vp, _vp,
                                           _vp, _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t,
                                           ctypes.POINTER(Debug), _vp]),
    "dash_attn_bwd_status": (ctypes.c_int, [_vp, _vp]),
    "dash_status_query": (ctypes.c_int, [_vp]),
    "dash_attn_bwd_noalloc": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, _vp, _vp, _vp,
                                             _vp, _vp, _vp, _vp, _vp, _vp, _vp]),
    "dash_schedule_tables": (ctypes.c_int, [_i32, _i32, ctypes.c_int, _ip, _ip, _ip, _ip, _ip]),
    "dash_schedule_predict": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, _i32, _dp,
                                             _dp]),
    "dash_attn_bwd_predict": (ctypes.c_int, [ctypes.POINTER(Desc), ctypes.c_int, _i32, _dp, _dp,
                                             _ip]),
    "dash_attn_bwd_resolve_schedule": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int,
                                                      ctypes.POINTER(ctypes.c_int)]),
    "dash_attn_schedule_tables": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, _i32, _ip, _ip,
                                                 _ip, _ip, _ip, ctypes.c_void_p, _ip]),
    "dash_attn_schedule_predict": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_int, _i32, _i32, _dp,
                                                  _dp]),
    "dash_attn_bwd_tune": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _vp, _vp, _vp, _vp, _vp,
                                          _vp, _vp, _vp, _vp, ctypes.c_size_t, _i32,
                                          ctypes.POINTER(ctypes.c_int), _vp, _vp]),
    "dash_attn_bwd_calibrate": (ctypes.c_int, [ctypes.POINTER(Desc), _vp, _vp, _vp, _vp, _vp,
                                               _vp, _vp, _vp, _vp, _vp, ctypes.c_size_t, _i32,
                                               _dp, _dp, _vp, _vp]),
    "dash_attn_bwd_costs": (ctypes.c_int, [ctypes.c_void_p, _dp]),
    "dash_schedule_fit_costs": (ctypes.c_int, [ctypes.c_void_p, _i32, _dp, _dp, _dp, _dp]),
    "dash_schedule_choose": (ctypes.c_int, [_i32, _i32, _i32, _i32, _dp,
                                            ctypes.POINTER(ctypes.c_int), _dp]),
    "dash_dag_longest_path": (ctypes.c_int, [_i32, _dp, _i32, _ip, _ip, _dp, _dp, _dp]),
    "dash_litmus_ordered_add": (ctypes.c_int, [_i32, _i32, _vp, _vp, _vp, _vp, ctypes.c_uint32,
                                               _vp]),
}

_LIB = None


def header_symbols(path: str = HEADER):
    """Function names declared in include/dash_attn.h."""
    with open(path) as f:
        text = f.read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(dash_[a-z0-9_]+)\s*\(", text)))


def load():
    """Load the shared library once; raise if it has not been built."""
    global _LIB
    if _LIB is not None:
        return _LIB
    if not os.path.exists(LIB_PATH):
        raise ImportError(
            f"{LIB_PATH} is missing: build it with "
            "`python -m deterministic_attention_backward_attn_amd.build` (hipcc, gfx950)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in _SIGS.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _LIB = lib
    return lib


def check(code: int, where: str):
    if code != 0:
        raise DashError(code, where)
