"""ctypes loader for libsta.so (argument marshalling only).

Loading fails loudly when the library has not been built: there is no
fallback of any kind.
"""

from __future__ import annotations

import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsta.so")
# The same library built with the kernels' bounds checks (-DSTA_DEBUG).
DEBUG_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libsta_debug.so")

STA_OK, STA_ERR_ARG, STA_ERR_SHAPE, STA_ERR_UNSUPPORTED, STA_ERR_ALLOC, STA_ERR_HIP = 0, -1, -2, -3, -4, -5
STA_BF16, STA_F32 = 0, 1
STA_LAYOUT_NATURAL, STA_LAYOUT_TILE_MAJOR = 0, 1
STA_PLAN_PARTIAL_TILES = 1


class PlanInfo(ctypes.Structure):
    _fields_ = [
        ("batch", ctypes.c_int32), ("heads", ctypes.c_int32), ("T", ctypes.c_int32),
        ("H", ctypes.c_int32), ("W", ctypes.c_int32), ("head_dim", ctypes.c_int32),
        ("tile", ctypes.c_int32 * 3), ("grid", ctypes.c_int32 * 3),
        ("tile_tokens", ctypes.c_int32), ("n_tiles", ctypes.c_int32),
        ("tokens", ctypes.c_int64), ("pairs", ctypes.c_int64), ("flops", ctypes.c_double),
        ("work_items", ctypes.c_int64), ("queries_per_item", ctypes.c_int32),
        ("kernel_variant", ctypes.c_int32), ("bwd_supported", ctypes.c_int32),
        ("bwd_queries_per_item", ctypes.c_int32), ("bwd_keys_per_item", ctypes.c_int32),
        ("bwd_items_dq", ctypes.c_int64),
        ("bwd_items_dkdv", ctypes.c_int64), ("partial_tiles", ctypes.c_int32),
        ("swa", ctypes.c_int32), ("split_items", ctypes.c_int32), ("pieces", ctypes.c_int32),
        ("scratch_bytes", ctypes.c_int64), ("launch_blocks", ctypes.c_int64),
    ]


_P = ctypes.c_void_p
_I = ctypes.c_int
_I64 = ctypes.c_int64
_IP = ctypes.POINTER(ctypes.c_int)
_I32P = ctypes.POINTER(ctypes.c_int32)

# name -> (restype, argtypes); every function declared in include/sta.h
SIGNATURES = {
    "sta_plan_create": (_I, [_I, _I, _I, _I, _I, _IP, _IP, _I, ctypes.POINTER(_P)]),
    "sta_plan_destroy": (_I, [_P]),
    "sta_plan_create_ex": (_I, [_I, _I, _I, _I, _I, _IP, _IP, _I, _I, ctypes.POINTER(_P)]),
    "sta_swa_plan_create": (_I, [_I, _I, _I, _I, _I, _IP, _IP, _I, ctypes.POINTER(_P)]),
    "sta_plan_get_info": (_I, [_P, ctypes.POINTER(PlanInfo)]),
    "sta_plan_perm": (_I, [_P, _I32P, _I64]),
    "sta_plan_kv_tiles": (_I, [_P, _I, _I, _I32P, _I, _IP]),
    "sta_plan_schedule": (_I, [_P, _I32P, _I64, ctypes.POINTER(_I64)]),
    "sta_plan_pieces": (_I, [_P, _I32P, _I64, ctypes.POINTER(_I64)]),
    "sta_plan_group_lists": (_I, [_P, _I32P, _I64, ctypes.POINTER(_I64)]),
    "sta_plan_q_tiles": (_I, [_P, _I, _I, _I32P, _I, _IP]),
    "sta_plan_walk": (_I, [_P, _I, _I, _I, _I32P, _I, _IP]),
    "sta_debug_flags": (_I, [ctypes.POINTER(ctypes.c_uint32), _I]),
    "sta_plan_schedule_bwd": (_I, [_P, _I, _I32P, _I64, ctypes.POINTER(_I64)]),
    "sta_tile_reorder": (_I, [_P, _P, _P, _I, _P]),
    "sta_tile_unreorder": (_I, [_P, _P, _P, _I, _P]),
    "sta_forward_plan": (_I, [_P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P]),
    "sta_forward_plan_lse": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P]),
    "sta_forward_plan_noalloc": (_I, [_P, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I, _P]),
    "sta_backward_plan": (_I, [_P, _P, _P, _P, _P, _P, _P, _P, _P, _P, _P, ctypes.c_float, _I, _I, _I,
                               _I, _P]),
    "sta_forward": (_I, [_P, _P, _P, _P, _I, _I, _I, _I, _I, _IP, _IP, _I, ctypes.c_float,
                         _I, _I, _I, _P]),
    "sta_window_errors": (_I, [_P, _P, _P, _I, _I, _I, _I, _I, _IP, _I, ctypes.c_float, _I, _I, _IP, _I,
                               ctypes.POINTER(ctypes.c_double), _P]),
    "sta_window_search": (_I, [ctypes.POINTER(_P), ctypes.POINTER(_P), ctypes.POINTER(_P), _I, _I, _I, _I, _I,
                               _I, _IP, _I, ctypes.c_float, _I, _I, _IP, _I, ctypes.c_double,
                               ctypes.POINTER(ctypes.c_double), _IP, _P]),
    "sta_window_select": (_I, [_I, _IP, _IP, _I, ctypes.POINTER(ctypes.c_double), ctypes.c_double, _IP]),
    "sta_window_candidates": (_I, [_IP, _IP, _I, _IP]),
    "sta_clear_plan_cache": (_I, []),
    "sta_status_string": (ctypes.c_char_p, [_I]),
}

_lib = None


class StaError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {status_string(status)}")


def _load(path: str) -> ctypes.CDLL:
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with "
                           "`python -m sliding_tile_attention_sta_amd.build`")
    l = ctypes.CDLL(path)
    for name, (res, args) in SIGNATURES.items():
        f = getattr(l, name)
        f.restype = res
        f.argtypes = args
    return l


def lib() -> ctypes.CDLL:
    global _lib
    if _lib is None:
        _lib = _load(LIB_PATH)
    return _lib


_debug_lib = None


def debug_lib() -> ctypes.CDLL:
    """libsta_debug.so: the same entry points with bounds-checked kernels
    (read the violations with sta_debug_flags)."""
    global _debug_lib
    if _debug_lib is None:
        _debug_lib = _load(DEBUG_LIB_PATH)
    return _debug_lib


def status_string(status: int) -> str:
    return lib().sta_status_string(status).decode()


def check(status: int, where: str) -> None:
    if status != STA_OK:
        raise StaError(status, where)
